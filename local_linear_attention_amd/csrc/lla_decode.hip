// Parallax decode step with a caller-supplied probe: one query per (batch, head) against a
// key-value cache of L positions, all of them in the query's prefix:
//
//   o = vbar - Sigma_KV rho,  p_j = softmax_j(q . k_j / h),  vbar = E_p[v],
//   Sigma_KV = E_p[(v - vbar)(k - kbar)^T]
//
// ("Parallax" blog post, section 2 "Parallax" for the forward equation; section 3
// "Optimized Decode Kernel" and Appendix C for the decode setting and its split over the
// key-value loop.)  Decode moves the whole cache once per step and does 8d flops per cached
// position, so it is bound by HBM, not by arithmetic: the kernels use the vector ALUs in
// fp32 (no matrix cores: a single query row would leave 15 of 16 MFMA columns idle, and the
// value operand would need a transposed copy of the cache), and the design goal is to keep
// enough loads in flight to stream the cache at full bandwidth.
//
//   lla_parallax_decode_kernel  block = 256 threads per (head, chunk of C keys): the chunk's
//                               scores s1 = q.k (log2 units) and probe scores
//                               t = rho.(k - q), both to LDS; the chunk max m; weights
//                               P1 = 2^(s1 - m), P2 = P1 t and their sums d1, d2; then
//                               O1 = sum P1 v, O2 = sum P2 v.  With one chunk per head the
//                               result is written directly, o = O1/d1 - (O2/d1 - (O1/d1)(d2/d1));
//                               otherwise (m, d1, d2, O1, O2) go to the workspace.
//   lla_parallax_merge_kernel   one block per head: rescales the chunks' partial sums to the
//                               largest chunk max (2^(m_s - M)) and merges them as above
//                               (the blog's Appendix C, item 3, with a separate launch).
// The probe scores are taken relative to rho . q (t = rho . (k - q)): a constant shift of
// the probe scores cancels in the merge, and this one is the same in every chunk of a head.
#include "lla_device.h"
#include "lla_internal.h"

#include <math.h>

#include <mutex>
#include <type_traits>
#include <utility>

namespace lla {
namespace {

constexpr int DC_THREADS = 256;
constexpr int DC_CMAX = 2048;   // keys per chunk at most (scores and weights in LDS)
constexpr float DC_LOG2E = 1.4426950408889634f;

__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void load8(const uint16_t* p, float (&x)[8]) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16));
}


// fp64 moments for fp32 inputs and for caches shorter than 2d, fp32 moments otherwise.
bool lla_decode_fp64(int dtype, int64_t L, int64_t d) { return dtype == 0 || L < 2 * d; }

template <int G>
__device__ __forceinline__ float group_sum(float x) {   // over G consecutive lanes
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// Block-wide max or sum of one float per thread (every thread gets the result).
__device__ __forceinline__ float block_reduce(float x, bool is_max, float* red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float y = __shfl_xor(x, o);
        x = is_max ? fmaxf(x, y) : x + y;
    }
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = x;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < DC_THREADS / 64; ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
    return r;
}

template <int D>
constexpr int dc_smem_floats() {
    // scores and weights of a chunk, later reused for the per-key-lane value sums
    return 2 * DC_CMAX > 2 * (DC_THREADS / (D / 8)) * (D + 1) ? 2 * DC_CMAX : 2 * (DC_THREADS / (D / 8)) * (D + 1);
}

template <typename TIn, int D>
__global__ __launch_bounds__(DC_THREADS) void lla_parallax_decode_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v, const TIn* __restrict__ rho,
    float* __restrict__ out, float* __restrict__ part, int L, int S, int C, float sl2) {
    constexpr int G = D / 8;               // threads per key, 8 features each
    constexpr int KPP = DC_THREADS / G;    // keys per pass
    __shared__ float sm[dc_smem_floats<D>()];
    __shared__ float red[DC_THREADS / 64];
    float* sx = sm;             // per key: s1 (log2 units), then P1
    float* sp = sm + DC_CMAX;   // per key: t, then P2
    const int tid = threadIdx.x, fg = tid % G, kl = tid / G;
    const int bh = static_cast<int>(blockIdx.x) / S, sidx = static_cast<int>(blockIdx.x) % S;
    const int j0 = sidx * C;
    const int cnt = min(L, j0 + C) - j0;   // >= 1: the host sizes chunks so that none is empty
    const TIn* kh = k + (static_cast<int64_t>(bh) * L + j0) * D + 8 * fg;
    const TIn* vh = v + (static_cast<int64_t>(bh) * L + j0) * D + 8 * fg;

    float qv[8], rv[8];
    load8(q + static_cast<int64_t>(bh) * D + 8 * fg, qv);
    load8(rho + static_cast<int64_t>(bh) * D + 8 * fg, rv);
    float cp = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) cp = fmaf(rv[e], qv[e], cp);
    const float c = group_sum<G>(cp);   // rho . q

    // Scores of the chunk's keys: key jj on the G lanes kl*G .. kl*G + G-1.
    float mloc = -INFINITY;
#pragma unroll 4
    for (int jj = kl; jj < cnt; jj += KPP) {
        float kv[8];
        load8(kh + static_cast<int64_t>(jj) * D, kv);
        float a = 0.0f, b = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a = fmaf(qv[e], kv[e], a);
            b = fmaf(rv[e], kv[e], b);
        }
        a = group_sum<G>(a);
        b = group_sum<G>(b);
        const float x = a * sl2;
        if (fg == 0) {
            sx[jj] = x;
            sp[jj] = b - c;
        }
        mloc = fmaxf(mloc, x);
    }
    const float m = block_reduce(mloc, true, red);   // also publishes sx, sp

    float d1l = 0.0f, d2l = 0.0f;
    for (int jj = tid; jj < cnt; jj += DC_THREADS) {
        const float e = exp2f(sx[jj] - m);
        const float et = e * sp[jj];
        sx[jj] = e;
        sp[jj] = et;
        d1l += e;
        d2l += et;
    }
    const float d1 = block_reduce(d1l, false, red);
    const float d2 = block_reduce(d2l, false, red);

    float o1[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, o2[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int jj = kl; jj < cnt; jj += KPP) {
        float vv[8];
        load8(vh + static_cast<int64_t>(jj) * D, vv);
        const float p1 = sx[jj], p2 = sp[jj];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            o1[e] = fmaf(p1, vv[e], o1[e]);
            o2[e] = fmaf(p2, vv[e], o2[e]);
        }
    }
    __syncthreads();   // the weights are no longer read: reuse their LDS for the value sums
    float* o1s = sm;
    float* o2s = sm + KPP * (D + 1);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        o1s[kl * (D + 1) + 8 * fg + e] = o1[e];
        o2s[kl * (D + 1) + 8 * fg + e] = o2[e];
    }
    __syncthreads();
    if (tid < D) {
        float O1 = 0.0f, O2 = 0.0f;
        for (int l = 0; l < KPP; ++l) {
            O1 += o1s[l * (D + 1) + tid];
            O2 += o2s[l * (D + 1) + tid];
        }
        if (S == 1) {
            const float inv = 1.0f / d1, ob = O1 * inv;
            out[static_cast<int64_t>(bh) * D + tid] = ob - (O2 * inv - ob * (d2 * inv));
        } else {
            float* pp = part + (static_cast<int64_t>(bh) * S + sidx) * (4 + 2 * D);
            pp[4 + tid] = O1;
            pp[4 + D + tid] = O2;
            if (tid == 0) {
                pp[0] = m;
                pp[1] = d1;
                pp[2] = d2;
                pp[3] = 0.0f;
            }
        }
    }
}

// One block per head.  Thread (chunk lane cl, feature f) sums every (256/D)-th chunk's
// rescaled value sums of feature f; the chunk lanes are then added through LDS.  Every load
// of the loop is independent of the others, so they overlap.
template <int D>
__global__ __launch_bounds__(DC_THREADS) void lla_parallax_merge_kernel(const float* __restrict__ part,
                                                                        float* __restrict__ out, int S) {
    constexpr int CL = DC_THREADS / D;   // chunk lanes
    constexpr int PST = 4 + 2 * D;       // floats per chunk
    __shared__ float red[DC_THREADS / 64];
    __shared__ float acc[CL][2 * D + 2];
    const int bh = static_cast<int>(blockIdx.x), tid = threadIdx.x, f = tid % D, cl = tid / D;
    const float* pb = part + static_cast<int64_t>(bh) * S * PST;
    float mx = -INFINITY;
    for (int s = tid; s < S; s += DC_THREADS) mx = fmaxf(mx, pb[static_cast<int64_t>(s) * PST]);
    const float M = block_reduce(mx, true, red);
    float d1 = 0.0f, d2 = 0.0f, O1 = 0.0f, O2 = 0.0f;
#pragma unroll 4
    for (int s = cl; s < S; s += CL) {
        const float* pp = pb + static_cast<int64_t>(s) * PST;
        const float w = exp2f(pp[0] - M);
        d1 = fmaf(w, pp[1], d1);
        d2 = fmaf(w, pp[2], d2);
        O1 = fmaf(w, pp[4 + f], O1);
        O2 = fmaf(w, pp[4 + D + f], O2);
    }
    acc[cl][f] = O1;
    acc[cl][D + f] = O2;
    if (f == 0) {
        acc[cl][2 * D] = d1;
        acc[cl][2 * D + 1] = d2;
    }
    __syncthreads();
    if (tid < D) {
        float a1 = 0.0f, a2 = 0.0f, s1 = 0.0f, s2 = 0.0f;
#pragma unroll
        for (int l = 0; l < CL; ++l) {
            a1 += acc[l][tid];
            a2 += acc[l][D + tid];
            s1 += acc[l][2 * D];
            s2 += acc[l][2 * D + 1];
        }
        const float inv = 1.0f / s1, ob = a1 * inv;
        out[static_cast<int64_t>(bh) * D + tid] = ob - (a2 * inv - ob * (s2 * inv));
    }
}

// Chunks per head: enough blocks to keep the chip's loads in flight (about 1024), chunks of
// at least 256 keys and at most DC_CMAX; no chunk is empty.
void decode_split(int64_t BH, int64_t L, int* S, int* C) {
    int64_t s = (1024 + BH - 1) / BH;
    s = s < 1 ? 1 : s;
    const int64_t by_len = (L + 255) / 256;
    if (s > by_len) s = by_len;
    const int64_t min_s = (L + DC_CMAX - 1) / DC_CMAX;
    if (s < min_s) s = min_s;
    const int64_t c = (L + s - 1) / s;
    *C = static_cast<int>(c);
    *S = static_cast<int>((L + c - 1) / c);
}

template <typename TIn, int D>
hipError_t launch_decode_t(const Problem& p, void* workspace) {
    const int64_t BH = p.B * p.H;
    int S = 1, C = 1;
    decode_split(BH, p.n, &S, &C);
    const float sl2 = static_cast<float>(DC_LOG2E / p.h);
    float* part = static_cast<float*>(workspace);
    prof_begin(p.stream, "lla_parallax_decode_kernel");
    lla_parallax_decode_kernel<TIn, D><<<dim3(static_cast<unsigned>(BH * S)), dim3(DC_THREADS), 0, p.stream>>>(
        static_cast<const TIn*>(p.q), static_cast<const TIn*>(p.k), static_cast<const TIn*>(p.v),
        static_cast<const TIn*>(p.rho), p.out, part, static_cast<int>(p.n), S, C, sl2);
    prof_end(p.stream);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || S == 1) return err;
    prof_begin(p.stream, "lla_parallax_merge_kernel");
    lla_parallax_merge_kernel<D><<<dim3(static_cast<unsigned>(BH)), dim3(DC_THREADS), 0, p.stream>>>(part, p.out, S);
    prof_end(p.stream);
    return hipGetLastError();
}

template <typename TIn>
hipError_t launch_decode_d(const Problem& p, void* workspace) {
    switch (p.d) {
        case 16: return launch_decode_t<TIn, 16>(p, workspace);
        case 32: return launch_decode_t<TIn, 32>(p, workspace);
        case 64: return launch_decode_t<TIn, 64>(p, workspace);
        case 128: return launch_decode_t<TIn, 128>(p, workspace);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t decode_workspace_bytes(int64_t B, int64_t H, int64_t L, int64_t d) {
    int S = 1, C = 1;
    decode_split(B * H, L, &S, &C);
    if (S == 1) return 0;
    return static_cast<size_t>(B * H * S * (4 + 2 * d) * 4);
}

hipError_t launch_parallax_decode(const Problem& p, void* workspace) {
    return p.dtype == 0 ? launch_decode_d<float>(p, workspace) : launch_decode_d<uint16_t>(p, workspace);
}

// =======================================================================================
// LLA decode step: b = vbar - C_vk (C_kk + lambda e^{-m} I)^{-1} (kbar - q) over each head's
// whole cache -- the LLA row of the "Parallax" blog post, section 2 "Canonical Formulation"
// (centred form of its Appendix E), for the newest position.  Launches:
//   lla_decode_stats_kernel    per chunk: scores x = q.k log2e/h (kept per key when the
//                              moments use split operands), chunk max m_c,
//                              omega_c = sum 2^(x - m_c), S_k,c = sum 2^(x - m_c) k;
//   lla_decode_moments_kernel  per chunk: the head's max M, omega and kbar from the chunk
//                              statistics; weights w = 2^(x - M); 64-key sub-tiles staged
//                              in LDS feature-major as R_k = sqrt(w)(k - kbar), R_v = sqrt(w) v;
//                              C_kk (upper 16x16 blocks) += R_k R_k^T and C_vk += R_v R_k^T on
//                              the matrix cores (fp64 16x16x4); S_v = sum w v; for bf16 inputs
//                              and caches of at least 2d positions
//                              lla_decode_moments_split_kernel instead (fp32 moments from bf16
//                              split operands, below);
//   lla_decode_reduce_kernel   (several chunks per head) the chunks' moments summed in fp64;
//   lla_decode_solve_kernel    per head: adds the ridge lambda 2^-M to the diagonal,
//                              Gauss-Jordan in registers (fp64), solves for y and writes
//                              b = S_v/omega - C_vk y.
// C_vk needs no centring of v: sum_j w_j (k_j - kbar) = 0 makes sum_j w_j vbar (k_j - kbar)^T
// vanish.  Moments in fp64 for fp32 inputs and for caches shorter than 2d (where the ridge
// alone conditions the solve); in fp32 otherwise.
namespace {

typedef double double4v __attribute__((ext_vector_type(4)));
typedef float float4x __attribute__((ext_vector_type(4)));

template <typename TA> struct Acc4;
template <> struct Acc4<double> { using type = double4v; };

__device__ __forceinline__ double4v mfma4(double a, double b, double4v c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}
// Row of the 16x16 output block held in register r of lane (g, c) (column c): the fp64
// instruction places rows 4r + g (the bf16 16x16x32 one of the split kernel, 4g + r).
template <typename TA> __device__ __forceinline__ int acc_row(int g, int r);
template <> __device__ __forceinline__ int acc_row<double>(int g, int r) { return 4 * r + g; }

constexpr int LD_SUB = 64;             // keys per staged sub-tile
constexpr int LD_LDW = LD_SUB + 2;     // row stride of the feature-major stage (elements)

// Blocks of a chunk's moments: the upper 16x16 blocks (I <= J) of C_kk row by row, then the
// NB x NB blocks of C_vk.
template <int D>
struct MomBlocks {
    static constexpr int NB = D / 16, NKK = NB * (NB + 1) / 2, NT = NKK + NB * NB;
    static constexpr int kind(int b) { return b < NKK ? 0 : 1; }
    static constexpr int I(int b) {
        if (b >= NKK) return (b - NKK) / NB;
        int i = 0, r = b;
        while (r >= NB - i) { r -= NB - i; ++i; }
        return i;
    }
    static constexpr int J(int b) {
        if (b >= NKK) return (b - NKK) % NB;
        int i = 0, r = b;
        while (r >= NB - i) { r -= NB - i; ++i; }
        return i + r;
    }
};

// acc[t] += op(block B0 + t) for t in Bs, with every block's rows and kind fixed at compile
// time (so the operand arrays stay in registers).
template <int D, int B0, typename TA, typename AccT, int N, int... Bs>
__device__ __forceinline__ void mfma_blocks(const TA (&ak)[D / 16], const TA (&av)[D / 16], AccT (&acc)[N],
                                            std::integer_sequence<int, Bs...>) {
    using MB = MomBlocks<D>;
    ((acc[Bs] = mfma4(std::integral_constant<int, MB::kind(B0 + Bs)>::value == 0
                          ? ak[std::integral_constant<int, MB::I(B0 + Bs)>::value]
                          : av[std::integral_constant<int, MB::I(B0 + Bs)>::value],
                      ak[std::integral_constant<int, MB::J(B0 + Bs)>::value], acc[Bs])),
     ...);
}

// Chunks per head for the LLA decode kernels: about 1024 blocks in all, 512 to DC_CMAX keys
// per chunk (the moments written per chunk stay small next to the cache), none empty.
void lla_decode_split(int64_t BH, int64_t L, int* S, int* C) {
    int64_t s = (1024 + BH - 1) / BH;
    const int64_t by_len = (L + 511) / 512;
    if (s > by_len) s = by_len;
    const int64_t min_s = (L + DC_CMAX - 1) / DC_CMAX;
    if (s < min_s) s = min_s;
    if (s < 1) s = 1;
    const int64_t c = (L + s - 1) / s;
    *C = static_cast<int>(c);
    *S = static_cast<int>((L + c - 1) / c);
}

template <typename TIn, int D>
__global__ __launch_bounds__(DC_THREADS) void lla_decode_stats_kernel(const TIn* __restrict__ q,
                                                                      const TIn* __restrict__ k,
                                                                      double* __restrict__ stats,
                                                                      float* __restrict__ xsc, int L, int S, int C,
                                                                      float sl2) {
    constexpr int G = D / 8, KPP = DC_THREADS / G;
    __shared__ float red[DC_THREADS / 64];
    __shared__ float acc[KPP][D + 1];
    const int tid = threadIdx.x, fg = tid % G, kl = tid / G;
    const int bh = static_cast<int>(blockIdx.x) / S, sidx = static_cast<int>(blockIdx.x) % S;
    const int j0 = sidx * C;
    const int cnt = min(L, j0 + C) - j0;
    const TIn* kh = k + (static_cast<int64_t>(bh) * L + j0) * D + 8 * fg;
    float qv[8];
    load8(q + static_cast<int64_t>(bh) * D + 8 * fg, qv);
    // one read of the keys: each lane group keeps its own running max mt and rescales its
    // omega and key sum when the max grows (a select, not a branch: groups differ)
    float mt = -INFINITY, om = 0.0f;
    float sk[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int jj = kl; jj < cnt; jj += KPP) {
        float kv[8];
        load8(kh + static_cast<int64_t>(jj) * D, kv);
        float a = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) a = fmaf(qv[e], kv[e], a);
        const float x = group_sum<G>(a) * sl2;
        if (xsc != nullptr && fg == 0) xsc[static_cast<int64_t>(bh) * L + j0 + jj] = x;
        const float mn = fmaxf(mt, x);
        const float sc = exp2f(mt - mn);   // 0 on the group's first key
        const float w = exp2f(x - mn);
        om = fmaf(om, sc, w);
#pragma unroll
        for (int e = 0; e < 8; ++e) sk[e] = fmaf(sk[e], sc, w * kv[e]);
        mt = mn;
    }
    const float m = block_reduce(mt, true, red);   // cnt >= 1: finite
    const float sc = exp2f(mt - m);                // 0 for groups that saw no key
    const float omega = block_reduce(fg == 0 ? om * sc : 0.0f, false, red);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[kl][8 * fg + e] = sk[e] * sc;
    __syncthreads();
    double* st = stats + (static_cast<int64_t>(bh) * S + sidx) * (2 + D);
    if (tid < D) {
        double t = 0.0;
        for (int l = 0; l < KPP; ++l) t += acc[l][tid];
        st[2 + tid] = t;
    }
    if (tid == 0) {
        st[0] = m;
        st[1] = omega;
    }
}

// Block-wide max or sum of one double per thread (every thread gets the result).
__device__ __forceinline__ double block_reduce_d(double x, bool is_max, double* red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const double y = __shfl_xor(x, o);
        x = is_max ? fmax(x, y) : x + y;
    }
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    double r = red[0];
#pragma unroll
    for (int i = 1; i < DC_THREADS / 64; ++i) r = is_max ? fmax(r, red[i]) : r + red[i];
    return r;
}

// The head's max M, omega and kbar (relative to M, into LDS kbar[D]) from its S chunks'
// statistics, with the whole block: chunks over threads for M and omega, (feature, chunk
// slice) pairs for kbar.  sh: DC_THREADS doubles of LDS.  Ends with a barrier.
template <int D>
__device__ __forceinline__ void head_stats(const double* __restrict__ hs, int S, double* sh, double* kbar,
                                           double* M_out, double* om_out) {
    constexpr int SL = DC_THREADS / D;
    const int tid = threadIdx.x;
    double m = -INFINITY;
    for (int s = tid; s < S; s += DC_THREADS) m = fmax(m, hs[s * (2 + D)]);
    const double M = block_reduce_d(m, true, sh);
    double o = 0.0;
    for (int s = tid; s < S; s += DC_THREADS) o += hs[s * (2 + D) + 1] * exp2(hs[s * (2 + D)] - M);
    const double om = block_reduce_d(o, false, sh + 8);
    const int f = tid % D, sl = tid / D;
    double t = 0.0;
    for (int s = sl; s < S; s += SL) t += hs[s * (2 + D) + 2 + f] * exp2(hs[s * (2 + D)] - M);
    __syncthreads();
    sh[tid] = t;
    __syncthreads();
    if (tid < D) {
        double r = 0.0;
#pragma unroll
        for (int l = 0; l < SL; ++l) r += sh[l * D + tid];
        kbar[tid] = r / om;
    }
    __syncthreads();
    *M_out = M;
    *om_out = om;
}

template <int D, typename TA>
constexpr int mom_smem_bytes() {
    return (2 * D * LD_LDW + D) * static_cast<int>(sizeof(TA)) + (DC_THREADS / (D / 8)) * (D + 1) * 4;
}

// The whole chunk loop of wave W (its accumulator blocks are compile-time), so that the
// accumulators stay in registers; every wave runs the same staging and barriers.
template <typename TIn, int D, typename TA, int W>
__device__ __forceinline__ void moments_wave(const TIn* __restrict__ qh, const TIn* __restrict__ kh,
                                             const TIn* __restrict__ vh, TA* rk, TA* rv, const TA* kb, float* svs,
                                             float Mf, int j0, int jend, int fg, int kl, int g, int c, float sl2,
                                             TA* __restrict__ mo) {
    using MB = MomBlocks<D>;
    using AccT = typename Acc4<TA>::type;
    constexpr int G = D / 8, KPP = DC_THREADS / G;
    constexpr int B0 = W * MB::NT / 4, B1 = (W + 1) * MB::NT / 4;
    float qv[8];
    load8(qh, qv);
    TA kbl[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) kbl[e] = kb[8 * fg + e];
    float sv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    constexpr int NA = B1 > B0 ? B1 - B0 : 1;   // a wave may own no block (d = 16)
    AccT acc[NA];
#pragma unroll
    for (int t = 0; t < NA; ++t) acc[t] = AccT{0, 0, 0, 0};
    for (int js = j0; js < jend; js += LD_SUB) {
        // stage: key js + jj on lanes kl*G.. (all lanes take part in the sums; keys past the
        // chunk are zero rows)
#pragma unroll
        for (int p = 0; p < (LD_SUB + KPP - 1) / KPP; ++p) {
            const int jj = kl + KPP * p;
            const bool in = jj < LD_SUB && js + jj < jend;
            float kv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, vv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            if (in) {
                load8(kh + static_cast<int64_t>(js + jj) * D, kv);
                load8(vh + static_cast<int64_t>(js + jj) * D, vv);
            }
            float a = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) a = fmaf(qv[e], kv[e], a);
            const float x = group_sum<G>(a) * sl2;
            const float w = in ? exp2f(x - Mf) : 0.0f;
            const TA sw = sqrt(static_cast<TA>(w));
            if (jj < LD_SUB) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    rk[(8 * fg + e) * LD_LDW + jj] = in ? sw * (static_cast<TA>(kv[e]) - kbl[e]) : static_cast<TA>(0);
                    rv[(8 * fg + e) * LD_LDW + jj] = sw * static_cast<TA>(vv[e]);
                    sv[e] = fmaf(w, vv[e], sv[e]);
                }
            }
        }
        __syncthreads();
#pragma unroll 2
        for (int s4 = 0; s4 < LD_SUB / 4; ++s4) {
            TA ak[MB::NB], av[MB::NB];
#pragma unroll
            for (int I = 0; I < MB::NB; ++I) {
                ak[I] = rk[(16 * I + c) * LD_LDW + 4 * s4 + g];
                av[I] = rv[(16 * I + c) * LD_LDW + 4 * s4 + g];
            }
            if constexpr (B1 > B0) mfma_blocks<D, B0>(ak, av, acc, std::make_integer_sequence<int, B1 - B0>{});
        }
        __syncthreads();
    }
#pragma unroll
    for (int b = B0; b < B1; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) mo[b * 256 + acc_row<TA>(g, r) * 16 + c] = acc[b - B0][r];
#pragma unroll
    for (int e = 0; e < 8; ++e) svs[kl * (D + 1) + 8 * fg + e] = sv[e];
}

template <typename TIn, int D, typename TA>
__global__ __launch_bounds__(DC_THREADS, 1) void lla_decode_moments_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const double* __restrict__ stats, TA* __restrict__ mom, int L, int S, int C, float sl2) {
    using MB = MomBlocks<D>;
    constexpr int G = D / 8, KPP = DC_THREADS / G;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    TA* rk = reinterpret_cast<TA*>(lds);
    TA* rv = rk + D * LD_LDW;
    TA* kb = rv + D * LD_LDW;
    float* svs = reinterpret_cast<float*>(kb + D);
    __shared__ double sh[DC_THREADS];
    __shared__ double kbd[D];
    const int tid = threadIdx.x, fg = tid % G, kl = tid / G;
    const int lane = tid & 63, g = lane >> 4, c = lane & 15;
    const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bh = static_cast<int>(blockIdx.x) / S, sidx = static_cast<int>(blockIdx.x) % S;
    const int j0 = sidx * C;
    const int jend = min(L, j0 + C);
    double M, om;
    head_stats<D>(stats + static_cast<int64_t>(bh) * S * (2 + D), S, sh, kbd, &M, &om);
    if (tid < D) kb[tid] = static_cast<TA>(kbd[tid]);
    __syncthreads();
    const float Mf = static_cast<float>(M);
    const TIn* qh = q + static_cast<int64_t>(bh) * D + 8 * fg;
    const TIn* kh = k + static_cast<int64_t>(bh) * L * D + 8 * fg;
    const TIn* vh = v + static_cast<int64_t>(bh) * L * D + 8 * fg;
    TA* mo = mom + (static_cast<int64_t>(bh) * S + sidx) * (MB::NT * 256 + D);
    switch (wu) {
        case 0: moments_wave<TIn, D, TA, 0>(qh, kh, vh, rk, rv, kb, svs, Mf, j0, jend, fg, kl, g, c, sl2, mo); break;
        case 1: moments_wave<TIn, D, TA, 1>(qh, kh, vh, rk, rv, kb, svs, Mf, j0, jend, fg, kl, g, c, sl2, mo); break;
        case 2: moments_wave<TIn, D, TA, 2>(qh, kh, vh, rk, rv, kb, svs, Mf, j0, jend, fg, kl, g, c, sl2, mo); break;
        default: moments_wave<TIn, D, TA, 3>(qh, kh, vh, rk, rv, kb, svs, Mf, j0, jend, fg, kl, g, c, sl2, mo); break;
    }
    __syncthreads();
    if (tid < D) {
        double t = 0.0;
        for (int l = 0; l < KPP; ++l) t += svs[l * (D + 1) + tid];
        mo[MB::NT * 256 + tid] = static_cast<TA>(t);
    }
}

// ---- Moments from split bf16 operands (bf16 inputs, fp32 moments; one block per CU at d = 128).
// R_k = sqrt(w) (k - kbar) and R_v = sqrt(w) v are formed in fp32 from the stats pass's
// scores and split into M3_PARTS bf16 parts, r = h + l (16 significant bits together); a
// 16x16 block then takes the products hh, hl, lh on v_mfma_f32_16x16x32_bf16 (32 keys per
// instruction): the dropped terms are below 2^-16 of each product (with three parts and six
// products, 2^-24; measured 1.3 times slower for errors that the two-part form already keeps
// near 1e-5).  Staging per sub-tile of 64 keys: a thread takes 16-byte row pieces (8 features
// of one key, loaded a sub-tile ahead), forms their parts in fp32 and stores each part
// row-major, [part][K, V][key][D + 8], with one 16-byte store.  The MFMA operands want 8
// consecutive keys of one feature per lane; the LDS transpose read (ds_read_b64_tr_b16, two
// per operand) delivers them from the row-major image: in each group of 16 lanes, lane L
// gives 4 consecutive features of key L / 4 and receives one feature of 4 consecutive keys.
// Two images alternate, so the parts of sub-tile t + 1 are formed while the products of
// sub-tile t run, with one barrier per sub-tile.
typedef __bf16 bf16x8d __attribute__((ext_vector_type(8)));
typedef short short4x __attribute__((ext_vector_type(4)));
constexpr int M3_PARTS = 2;         // bf16 parts per operand (2: hi + lo; 3: hi + mid + lo)
// Keys per sub-tile: 32 (one MFMA step; four blocks per CU at d <= 64, two at d = 128), 64 at
// d = 16 (where 32 keys would leave threads without a piece).
template <int D>
constexpr int msp_sub() { return D == 16 ? 64 : 32; }

template <int D>
constexpr int msp_row() { return D + 8; }   // halves per key row of a part image
template <int D>
constexpr int msp_img_bytes() { return M3_PARTS * 2 * msp_sub<D>() * msp_row<D>() * 2; }   // [part][K, V][key][D + 8]
template <int D>
constexpr int msp_smem_bytes() { return 2 * msp_img_bytes<D>(); }

__device__ __forceinline__ float4x mfma_bf(bf16x8d a, bf16x8d b, float4x c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// c += a b for a, b given as M3_PARTS bf16 parts each, smallest products first: with three
// parts hh, hm, mh, hl, lh, mm (dropped terms below 2^-24 relative), with two hh, hl, lh
// (dropped terms below 2^-16).
__device__ __forceinline__ float4x mfma_split(const bf16x8d (&a)[M3_PARTS], const bf16x8d (&b)[M3_PARTS], float4x c) {
    if constexpr (M3_PARTS == 3) {
        c = mfma_bf(a[1], b[1], c);
        c = mfma_bf(a[2], b[0], c);
        c = mfma_bf(a[0], b[2], c);
    }
    c = mfma_bf(a[1], b[0], c);
    c = mfma_bf(a[0], b[1], c);
    return mfma_bf(a[0], b[0], c);
}

template <int D, int B0, int N, int... Bs>
__device__ __forceinline__ void mfma_split_blocks(const bf16x8d (&kop)[D / 16][M3_PARTS],
                                             const bf16x8d (&vop)[D / 16][M3_PARTS],
                                             float4x (&acc)[N], std::integer_sequence<int, Bs...>) {
    using MB = MomBlocks<D>;
    ((acc[Bs] = mfma_split(std::integral_constant<int, MB::kind(B0 + Bs)>::value == 0
                          ? kop[std::integral_constant<int, MB::I(B0 + Bs)>::value]
                          : vop[std::integral_constant<int, MB::I(B0 + Bs)>::value],
                      kop[std::integral_constant<int, MB::J(B0 + Bs)>::value], acc[Bs])),
     ...);
}

// MFMA operand from a row-major part image: lane (g, c) receives feature f0 + c of keys
// k0 + 8 g .. k0 + 8 g + 7 (elements are `RL` halves apart from key to key).
template <int RL>
__device__ __forceinline__ bf16x8d tr_operand(const unsigned char* part, int k0, int f0, int g, int c) {
    const short* p = reinterpret_cast<const short*>(part) + (k0 + 8 * g + (c >> 2)) * RL + f0 + 4 * (c & 3);
    typedef __attribute__((address_space(3))) short4x* lds_short4x;
    const short4x lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4x)(const_cast<short*>(p)));
    const short4x hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4x)(const_cast<short*>(p + 4 * RL)));
    return __builtin_bit_cast(bf16x8d, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Wave W of a block: the moment blocks [B0, B1) over keys [j0, jend), and this thread's
// partial sums S_v of its 8 features (8 (tid mod D/8) ..) in sv.
template <typename TIn, int D, int W>
__device__ __forceinline__ void moments_split_wave(const TIn* __restrict__ kh, const TIn* __restrict__ vh,
                                              const float* __restrict__ xh, const float* kbf, unsigned char* lds,
                                              float Mf, int j0, int jend, int tid, float* __restrict__ mo,
                                              float (&sv)[8]) {
    using MB = MomBlocks<D>;
    constexpr int NB = D / 16;
    constexpr int B0 = W * MB::NT / 4, B1 = (W + 1) * MB::NT / 4;
    constexpr int NA = B1 > B0 ? B1 - B0 : 1;
    constexpr int RL = msp_row<D>();
    constexpr int M3_SUB = msp_sub<D>();
    constexpr int PK = D / 8;                        // 16-byte pieces per key row
    constexpr int APIECES = M3_SUB * PK;             // pieces of K (then of V) per sub-tile
    constexpr int CPT = 2 * APIECES / DC_THREADS;    // pieces per thread
    constexpr int PART = 2 * M3_SUB * RL * 2;        // bytes per part image
    constexpr int VB = B0 > MB::NKK ? B0 : MB::NKK;
    constexpr int VI0 = B1 > MB::NKK ? MB::I(VB) : 0;
    constexpr int VI1 = B1 > MB::NKK ? MB::I(B1 - 1) : -1;
    static_assert(sizeof(TIn) == 2, "split-operand moments take bf16 inputs");
    static_assert(CPT >= 1 && (2 * APIECES) % DC_THREADS == 0 && DC_THREADS % PK == 0, "piece mapping");
    const int lane = tid & 63, g = lane >> 4, c = lane & 15;
    const int fc = tid % PK;                         // this thread's features 8 fc .. 8 fc + 7
    float kb8[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) kb8[t] = kbf[8 * fc + t];
    float4x acc[NA];
#pragma unroll
    for (int t = 0; t < NA; ++t) acc[t] = float4x{0.f, 0.f, 0.f, 0.f};
    uint4 pre[CPT];
    float xpre[CPT];
    // piece u = tid + 256 e: K (u < APIECES) or V, key (u mod APIECES) / PK, features 8 fc ..
    auto fetch = [&](int js) {
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
            const int u = tid + DC_THREADS * e;
            const int arr = u / APIECES, key = (u % APIECES) / PK;
            const int j = js + key;
            pre[e] = uint4{0u, 0u, 0u, 0u};
            xpre[e] = -INFINITY;
            if (j < jend) {
                pre[e] = *reinterpret_cast<const uint4*>((arr == 0 ? kh : vh) + static_cast<int64_t>(j) * D + 8 * fc);
                xpre[e] = xh[j];
            }
        }
    };
    auto stash = [&](unsigned char* img) {
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
            const int u = tid + DC_THREADS * e;
            const int arr = u / APIECES, key = (u % APIECES) / PK;
            const float sw = exp2f((xpre[e] - Mf) * 0.5f);
            const uint32_t wd[4] = {pre[e].x, pre[e].y, pre[e].z, pre[e].w};
            bf16x8d part[M3_PARTS];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const uint32_t w2 = wd[t >> 1];
                const float x = __uint_as_float((t & 1) ? (w2 & 0xffff0000u) : (w2 << 16));
                float r = sw * (x - (arr == 0 ? kb8[t] : 0.0f));
                if (arr == 1) sv[t] = fmaf(sw * sw, x, sv[t]);
#pragma unroll
                for (int lv = 0; lv < M3_PARTS; ++lv) {
                    const __bf16 hp = static_cast<__bf16>(r);
                    part[lv][t] = hp;
                    r -= static_cast<float>(hp);
                }
            }
#pragma unroll
            for (int lv = 0; lv < M3_PARTS; ++lv)
                *reinterpret_cast<bf16x8d*>(img + lv * PART + ((arr * M3_SUB + key) * RL + 8 * fc) * 2) = part[lv];
        }
    };
    auto products = [&](const unsigned char* img) {
        if constexpr (B1 > B0) {
#pragma unroll
            for (int ks = 0; ks < M3_SUB / 32; ++ks) {
                bf16x8d kop[NB][M3_PARTS], vop[NB][M3_PARTS];
#pragma unroll
                for (int R = 0; R < NB; ++R)
#pragma unroll
                    for (int lv = 0; lv < M3_PARTS; ++lv) kop[R][lv] = tr_operand<RL>(img + lv * PART, 32 * ks, 16 * R, g, c);
#pragma unroll
                for (int R = VI0; R <= VI1; ++R)
#pragma unroll
                    for (int lv = 0; lv < M3_PARTS; ++lv)
                        vop[R][lv] = tr_operand<RL>(img + lv * PART + M3_SUB * RL * 2, 32 * ks, 16 * R, g, c);
                mfma_split_blocks<D, B0>(kop, vop, acc, std::make_integer_sequence<int, B1 - B0>{});
            }
        }
    };
    // Sub-tile t's products read image t mod 2; meanwhile the parts of t + 1 go into the
    // other image (last read before the previous barrier) and the rows of t + 2 are loaded.
    const int nsub = (jend - j0 + M3_SUB - 1) / M3_SUB;
    unsigned char* img0 = lds;
    unsigned char* img1 = lds + msp_img_bytes<D>();
    fetch(j0);
    stash(img0);
    if (nsub > 1) fetch(j0 + M3_SUB);
    __syncthreads();
    for (int t = 0; t < nsub; ++t) {
        products((t & 1) ? img1 : img0);
        if (t + 1 < nsub) {
            stash(((t + 1) & 1) ? img1 : img0);
            if (t + 2 < nsub) fetch(j0 + (t + 2) * M3_SUB);
        }
        __syncthreads();
    }
#pragma unroll
    for (int b = B0; b < B1; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) mo[b * 256 + (4 * g + r) * 16 + c] = acc[b - B0][r];
}

template <typename TIn, int D>
__global__ __launch_bounds__(DC_THREADS, D <= 64 ? 4 : 2) void lla_decode_moments_split_kernel(
    const TIn* __restrict__ k, const TIn* __restrict__ v, const double* __restrict__ stats,
    const float* __restrict__ xsc, float* __restrict__ mom, int L, int S, int C) {
    using MB = MomBlocks<D>;
    static_assert(D <= 128, "split-operand moments serve d <= 128");
    static_assert(DC_THREADS * 8 * 4 <= 2 * msp_img_bytes<D>(), "S_v partials fit in the images");
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    __shared__ double sh[DC_THREADS];
    __shared__ double kbd[D];
    __shared__ float kbf[D];
    const int tid = threadIdx.x;
    const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bh = static_cast<int>(blockIdx.x) / S, sidx = static_cast<int>(blockIdx.x) % S;
    const int j0 = sidx * C;
    const int jend = min(L, j0 + C);
    double M, om;
    head_stats<D>(stats + static_cast<int64_t>(bh) * S * (2 + D), S, sh, kbd, &M, &om);
    if (tid < D) kbf[tid] = static_cast<float>(kbd[tid]);
    __syncthreads();
    const float Mf = static_cast<float>(M);
    const TIn* kh = k + static_cast<int64_t>(bh) * L * D;
    const TIn* vh = v + static_cast<int64_t>(bh) * L * D;
    const float* xh = xsc + static_cast<int64_t>(bh) * L;
    float* mo = mom + (static_cast<int64_t>(bh) * S + sidx) * (MB::NT * 256 + D);
    float sv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    switch (wu) {
        case 0: moments_split_wave<TIn, D, 0>(kh, vh, xh, kbf, lds, Mf, j0, jend, tid, mo, sv); break;
        case 1: moments_split_wave<TIn, D, 1>(kh, vh, xh, kbf, lds, Mf, j0, jend, tid, mo, sv); break;
        case 2: moments_split_wave<TIn, D, 2>(kh, vh, xh, kbf, lds, Mf, j0, jend, tid, mo, sv); break;
        default: moments_split_wave<TIn, D, 3>(kh, vh, xh, kbf, lds, Mf, j0, jend, tid, mo, sv); break;
    }
    // S_v: every thread's partial sums of its 8 features, through the (now free) images.
    float* svp = reinterpret_cast<float*>(lds);   // [thread][8]
    *reinterpret_cast<float4x*>(svp + tid * 8) = float4x{sv[0], sv[1], sv[2], sv[3]};
    *reinterpret_cast<float4x*>(svp + tid * 8 + 4) = float4x{sv[4], sv[5], sv[6], sv[7]};
    __syncthreads();
    if (tid < D) {
        constexpr int PK = D / 8;
        float t = 0.0f;
        for (int th = tid / 8; th < DC_THREADS; th += PK) t += svp[th * 8 + (tid & 7)];
        mo[MB::NT * 256 + tid] = t;
    }
}

// Sum of the S chunks' moments of each head, in chunk order (fp64): one thread per entry.
template <typename TA>
__global__ __launch_bounds__(DC_THREADS) void lla_decode_reduce_kernel(const TA* __restrict__ mom,
                                                                       double* __restrict__ sum, int S, int E,
                                                                       int blocks_per_head) {
    const int bh = static_cast<int>(blockIdx.x) / blocks_per_head;
    const int e = (static_cast<int>(blockIdx.x) % blocks_per_head) * DC_THREADS + static_cast<int>(threadIdx.x);
    if (e >= E) return;
    const TA* p = mom + static_cast<int64_t>(bh) * S * E + e;
    double t0 = 0.0, t1 = 0.0, t2 = 0.0, t3 = 0.0;
    int s = 0;
    for (; s + 4 <= S; s += 4) {
        t0 += static_cast<double>(p[static_cast<int64_t>(s) * E]);
        t1 += static_cast<double>(p[static_cast<int64_t>(s + 1) * E]);
        t2 += static_cast<double>(p[static_cast<int64_t>(s + 2) * E]);
        t3 += static_cast<double>(p[static_cast<int64_t>(s + 3) * E]);
    }
    for (; s < S; ++s) t0 += static_cast<double>(p[static_cast<int64_t>(s) * E]);
    sum[static_cast<int64_t>(bh) * E + e] = (t0 + t1) + (t2 + t3);
}

// Index of entry (i, j), i <= j, of C_kk in a head's moment blocks.
template <int D>
__device__ __forceinline__ int kk_index(int i, int j) {
    constexpr int NB = D / 16;
    const int I = i >> 4, J = j >> 4;
    return (I * NB - I * (I - 1) / 2 + (J - I)) * 256 + (i & 15) * 16 + (j & 15);
}

// Per head: A = C_kk + lambda 2^-M I (fp64), solved for y with A y = kbar - q by Gauss-Jordan
// elimination: thread (ti, tj) of a 16 x 16 grid holds the TS x TS tile of A at rows
// ti*TS.., columns tj*TS.. in registers; step p publishes column p (double-buffered in LDS,
// one barrier per step) and every thread eliminates it from its rows other than p.  On the
// symmetric trailing block row p equals column p, and the columns of earlier pivots are
// already zero in row p, so column p alone drives the update.  The pivots are those of
// LDL^T; a pivot that is not positive (lambda > 0: made so by rounding) or below 1e-12 of the
// largest diagonal entry (lambda = 0: a direction the cache leaves undetermined) is skipped
// and its unknown set to 0.  Then b = S_v/omega - C_vk y.
// mom: the head's summed moments (TM = double) or, with one chunk per head, the chunk's own.
template <typename TIn, int D, typename TM>
__global__ __launch_bounds__(DC_THREADS) void lla_decode_solve_kernel(
    const TIn* __restrict__ q, const double* __restrict__ stats, const TM* __restrict__ mom,
    float* __restrict__ out, int S, double lambda) {
    using MB = MomBlocks<D>;
    constexpr int TS = D / 16, E = MB::NT * 256 + D;
    __shared__ double sh[DC_THREADS];
    __shared__ double kbd[D];
    __shared__ double colb[2][D];
    __shared__ double zb[2];
    __shared__ double dg[D];
    __shared__ double ys[D];
    const int tid = threadIdx.x, bh = static_cast<int>(blockIdx.x);
    const int ti = tid >> 4, tj = tid & 15;
    double M, om;
    head_stats<D>(stats + static_cast<int64_t>(bh) * S * (2 + D), S, sh, kbd, &M, &om);
    const double ridge = lambda * exp2(-M);
    const TM* mh = mom + static_cast<int64_t>(bh) * E;
    double a[TS][TS];
    double dmax = 0.0;
#pragma unroll
    for (int ia = 0; ia < TS; ++ia)
#pragma unroll
        for (int ib = 0; ib < TS; ++ib) {
            const int i = ti * TS + ia, j = tj * TS + ib;
            a[ia][ib] = static_cast<double>(mh[i <= j ? kk_index<D>(i, j) : kk_index<D>(j, i)]) + (i == j ? ridge : 0.0);
            if (i == j) dmax = fmax(dmax, a[ia][ib]);
        }
    const double thr = lambda > 0.0 ? 0.0 : 1e-12 * block_reduce_d(dmax, true, sh);
    double z = tid < D ? kbd[tid] - load_f64(q, static_cast<int64_t>(bh) * D + tid) : 0.0;
    for (int pb = 0; pb < 16; ++pb) {
#pragma unroll
        for (int pp = 0; pp < TS; ++pp) {
            const int p = pb * TS + pp;
            double* cb = colb[p & 1];
            if (tj == pb) {
#pragma unroll
                for (int ia = 0; ia < TS; ++ia) cb[ti * TS + ia] = a[ia][pp];
            }
            if (tid == p) zb[p & 1] = z;
            __syncthreads();
            const double piv = cb[p];
            if (piv > thr) {
                // 1 / piv: the hardware reciprocal and two Newton steps (about 1 ulp)
                double f = __builtin_amdgcn_rcp(piv);
                f = fma(f, fma(-piv, f, 1.0), f);
                f = fma(f, fma(-piv, f, 1.0), f);
                double rp[TS];
#pragma unroll
                for (int ib = 0; ib < TS; ++ib) rp[ib] = tj * TS + ib > p ? cb[tj * TS + ib] : 0.0;
#pragma unroll
                for (int ia = 0; ia < TS; ++ia) {
                    const int i = ti * TS + ia;
                    const double cr = i == p ? 0.0 : cb[i] * f;
#pragma unroll
                    for (int ib = 0; ib < TS; ++ib) a[ia][ib] = fma(-cr, rp[ib], a[ia][ib]);
                }
                if (tid < D && tid != p) z = fma(-cb[tid] * f, zb[p & 1], z);
            }
            if (tid == 0) dg[p] = piv > thr ? piv : 0.0;
        }
    }
    __syncthreads();
    if (tid < D) ys[tid] = dg[tid] > 0.0 ? z / dg[tid] : 0.0;
    __syncthreads();
    // b_f = S_v,f / omega - sum_g C_vk[f][g] y_g; thread (slice sl, feature f)
    constexpr int SL = DC_THREADS / D;
    const int f = tid % D, sl = tid / D;
    double acc = 0.0;
    for (int gi = sl; gi < D; gi += SL) {
        const int e = (MB::NKK + (f >> 4) * MB::NB + (gi >> 4)) * 256 + (f & 15) * 16 + (gi & 15);
        acc = fma(static_cast<double>(mh[e]), ys[gi], acc);
    }
    sh[tid] = acc;
    __syncthreads();
    if (tid < D) {
        double t = 0.0;
#pragma unroll
        for (int l = 0; l < SL; ++l) t += sh[l * D + tid];
        out[static_cast<int64_t>(bh) * D + tid] = static_cast<float>(static_cast<double>(mh[MB::NT * 256 + tid]) / om - t);
    }
}

// Workspace: chunk statistics, then the chunks' moments, then (several chunks per head) the
// heads' summed moments; each region starts on a 256-byte boundary.
struct LlaDecodeLayout {
    int64_t stats_bytes, score_bytes, mom_bytes, sum_bytes;
};
// fp32 moments from split bf16 operands (they read the stats pass's scores): bf16 inputs
// with fp32 moments.
bool lla_decode_split_operands(int dtype, int64_t L, int64_t d) { return !lla_decode_fp64(dtype, L, d) && d <= 128; }
LlaDecodeLayout lla_decode_layout(int64_t BH, int64_t L, int64_t d, int dtype) {
    int S = 1, C = 1;
    lla_decode_split(BH, L, &S, &C);
    const int64_t nb = d / 16, e = (nb * (nb + 1) / 2 + nb * nb) * 256 + d;
    const int64_t ta = lla_decode_fp64(dtype, L, d) ? 8 : 4;
    auto up = [](int64_t x) { return (x + 255) & ~int64_t(255); };
    return {up(BH * S * (2 + d) * 8), lla_decode_split_operands(dtype, L, d) ? up(BH * L * 4) : 0, up(BH * S * e * ta),
            S > 1 ? BH * e * 8 : 0};
}

template <typename TIn, int D, typename TA>
hipError_t launch_lla_decode_t(const Problem& p, void* workspace) {
    using MB = MomBlocks<D>;
    constexpr int E = MB::NT * 256 + D;
    const int64_t BH = p.B * p.H;
    int S = 1, C = 1;
    lla_decode_split(BH, p.n, &S, &C);
    const float sl2 = static_cast<float>(DC_LOG2E / p.h);
    const LlaDecodeLayout lay = lla_decode_layout(BH, p.n, D, p.dtype);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    double* stats = reinterpret_cast<double*>(ws);
    float* xsc = lay.score_bytes > 0 ? reinterpret_cast<float*>(ws + lay.stats_bytes) : nullptr;
    TA* mom = reinterpret_cast<TA*>(ws + lay.stats_bytes + lay.score_bytes);
    double* msum = reinterpret_cast<double*>(ws + lay.stats_bytes + lay.score_bytes + lay.mom_bytes);
    // TA = float: bf16 inputs, split-operand moments; TA = double: the fp64 moments kernel.
    constexpr bool kSplit = std::is_same<TA, float>::value;
    static_assert(!kSplit || std::is_same<TIn, uint16_t>::value, "split-operand moments take bf16 inputs");
    static_assert(kSplit || mom_smem_bytes<D, TA>() <= 150 * 1024, "LDS");
    // The dynamic LDS limit, raised once per instantiation and device (the current one).
    static std::mutex attr_mu;
    static bool attr_done[64] = {};
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    {
        std::lock_guard<std::mutex> lock(attr_mu);
        if (!attr_done[dev]) {
            if constexpr (kSplit)
                err = hipFuncSetAttribute(reinterpret_cast<const void*>(&lla_decode_moments_split_kernel<TIn, D>),
                                          hipFuncAttributeMaxDynamicSharedMemorySize, msp_smem_bytes<D>());
            else
                err = hipFuncSetAttribute(reinterpret_cast<const void*>(&lla_decode_moments_kernel<TIn, D, TA>),
                                          hipFuncAttributeMaxDynamicSharedMemorySize, mom_smem_bytes<D, TA>());
            if (err != hipSuccess) return err;
            attr_done[dev] = true;
        }
    }
    const unsigned blocks = static_cast<unsigned>(BH * S);
    prof_begin(p.stream, "lla_decode_stats_kernel");
    lla_decode_stats_kernel<TIn, D><<<dim3(blocks), dim3(DC_THREADS), 0, p.stream>>>(
        static_cast<const TIn*>(p.q), static_cast<const TIn*>(p.k), stats, xsc, static_cast<int>(p.n), S, C, sl2);
    prof_end(p.stream);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    prof_begin(p.stream, "lla_decode_moments_kernel");
    if constexpr (kSplit)
        lla_decode_moments_split_kernel<TIn, D><<<dim3(blocks), dim3(DC_THREADS), msp_smem_bytes<D>(), p.stream>>>(
            static_cast<const TIn*>(p.k), static_cast<const TIn*>(p.v), stats, xsc, mom, static_cast<int>(p.n), S, C);
    else
        lla_decode_moments_kernel<TIn, D, TA><<<dim3(blocks), dim3(DC_THREADS), mom_smem_bytes<D, TA>(), p.stream>>>(
            static_cast<const TIn*>(p.q), static_cast<const TIn*>(p.k), static_cast<const TIn*>(p.v), stats, mom,
            static_cast<int>(p.n), S, C, sl2);
    prof_end(p.stream);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (S > 1) {
        const int bph = (E + DC_THREADS - 1) / DC_THREADS;
        prof_begin(p.stream, "lla_decode_reduce_kernel");
        lla_decode_reduce_kernel<TA><<<dim3(static_cast<unsigned>(BH * bph)), dim3(DC_THREADS), 0, p.stream>>>(
            mom, msum, S, E, bph);
        prof_end(p.stream);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        prof_begin(p.stream, "lla_decode_solve_kernel");
        lla_decode_solve_kernel<TIn, D, double><<<dim3(static_cast<unsigned>(BH)), dim3(DC_THREADS), 0, p.stream>>>(
            static_cast<const TIn*>(p.q), stats, msum, p.out, S, p.lambda);
    } else {
        prof_begin(p.stream, "lla_decode_solve_kernel");
        lla_decode_solve_kernel<TIn, D, TA><<<dim3(static_cast<unsigned>(BH)), dim3(DC_THREADS), 0, p.stream>>>(
            static_cast<const TIn*>(p.q), stats, mom, p.out, S, p.lambda);
    }
    prof_end(p.stream);
    return hipGetLastError();
}

template <typename TIn, int D>
hipError_t launch_lla_decode_p(const Problem& p, void* workspace) {
    if constexpr (std::is_same<TIn, uint16_t>::value)
        if (!lla_decode_fp64(p.dtype, p.n, D)) return launch_lla_decode_t<TIn, D, float>(p, workspace);
    return launch_lla_decode_t<TIn, D, double>(p, workspace);
}

template <typename TIn>
hipError_t launch_lla_decode_d(const Problem& p, void* workspace) {
    switch (p.d) {
        case 16: return launch_lla_decode_p<TIn, 16>(p, workspace);
        case 32: return launch_lla_decode_p<TIn, 32>(p, workspace);
        case 64: return launch_lla_decode_p<TIn, 64>(p, workspace);
        case 128: return launch_lla_decode_p<TIn, 128>(p, workspace);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t lla_decode_workspace_bytes(int64_t B, int64_t H, int64_t L, int64_t d, int dtype) {
    const LlaDecodeLayout lay = lla_decode_layout(B * H, L, d, dtype);
    return static_cast<size_t>(lay.stats_bytes + lay.score_bytes + lay.mom_bytes + lay.sum_bytes);
}

hipError_t launch_lla_decode(const Problem& p, void* workspace) {
    return p.dtype == 0 ? launch_lla_decode_d<float>(p, workspace) : launch_lla_decode_d<uint16_t>(p, workspace);
}

}  // namespace lla
