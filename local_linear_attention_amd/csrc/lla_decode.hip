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
#include "lla_internal.h"

#include <math.h>

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

}  // namespace lla
