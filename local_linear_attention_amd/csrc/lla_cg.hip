// Causal LLA forward with each query's linear system solved by conjugate gradient over its
// prefix, the solver the pages name for the exact forward ("Parallax" blog post, section 2
// "Difficulties in Scaling LLA": one system per query position, parallel CG, T iterations of
// an attention-like pass each, T L d memory accesses).  One workgroup per query row, fp64
// after the load:
//
//   pass 0   m = max_j q.k_j / h;  pass 1  wt_j = exp(q.k_j / h - m), omega, kbar, vbar
//   CG       A x = kbar - q with A = sum_j wt_j (k_j - kbar)(k_j - kbar)^T + lambda e^{-m} I
//            never formed: every iteration is one pass over the prefix,
//              A p = sum_j wt_j ((k_j - kbar) . p) (k_j - kbar) + lambda e^{-m} p,
//            then the usual CG updates (x from 0); it stops when |r| <= tol |kbar - q|, when
//            p.Ap is not positive, or after max_iter iterations
//   output   b = vbar - sum_j wt_j ((k_j - kbar) . x) (v_j - vbar)   (= vbar - C_vk x).
//   A row whose residual did not reach the tolerance is handed to the direct fp64 solve
//   (lla_exact_kernel in list mode, after this launch): CG needs about sqrt(cond A)
//   iterations, and a ridge lambda e^{-m} far below the spread of the weighted keys (sharp
//   weights, prefixes shorter than d) leaves cond A near 1e8, out of reach of a budget
//   proportional to d -- the ill-conditioning the pages name as CG's weakness.
//
// The same centred system as the direct fp64 path (lla_exact.hip), so both give the LLA
// intercept; this one keeps only d-vectors per query (no d x d state) at the price of one
// prefix pass per iteration.
#include "lla_device.h"
#include "lla_internal.h"

#include <math.h>

namespace lla {
namespace {


constexpr int CG_NT = 256;
constexpr int kCgMaxIterFactor = 4;   // at most 4d iterations (d suffice in exact arithmetic)
constexpr double kCgTol = 1e-10;      // stop at |r| <= kCgTol |kbar - q|

template <typename TIn, int D>
__global__ __launch_bounds__(CG_NT) void lla_cg_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                       const TIn* __restrict__ v, float* __restrict__ out, int n,
                                                       int BH, double inv_h, double lambda, int max_iter,
                                                       double tol, unsigned* __restrict__ count,
                                                       int* __restrict__ list) {
    constexpr int NT = CG_NT;
    constexpr int CHK = 2048 / D;   // keys per staged chunk (16 KiB of fp64 per array)
    constexpr int G = NT / CHK;     // threads per key in the dot products
    constexpr int DG = D / G;       // features per thread in them
    constexpr int KL = NT / D;      // key lanes of the per-feature sums
    constexpr int LD = D + 1;
    static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0 && D % G == 0 && NT % D == 0, "layout");

    __shared__ double qs[D], kbar[D], vbar[D], xs[D], ps[D];
    __shared__ double Ks[CHK * LD];
    __shared__ double Vs[CHK * LD];
    __shared__ double ws[CHK];
    __shared__ double part[NT];
    __shared__ double red[NT / 64];

    const int tid = threadIdx.x;
    const int i = n - 1 - static_cast<int>(blockIdx.x / BH);   // longest rows first
    const int bh = static_cast<int>(blockIdx.x % BH);
    const int64_t base = static_cast<int64_t>(bh) * n * D;
    const TIn* kh = k + base;
    const TIn* vh = v + base;
    const int cnt = i + 1;
    const int fa = tid % D, kl = tid / D;

    for (int e = tid; e < D; e += NT) qs[e] = load_f64(q + base, static_cast<int64_t>(i) * D + e);

    auto block_sum = [&](double x, bool is_max) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const double y = __shfl_xor(x, o);
            x = is_max ? fmax(x, y) : x + y;
        }
        __syncthreads();
        if ((tid & 63) == 0) red[tid >> 6] = x;
        __syncthreads();
        double r = red[0];
#pragma unroll
        for (int w = 1; w < NT / 64; ++w) r = is_max ? fmax(r, red[w]) : r + red[w];
        return r;
    };
    // Sum over the key lanes of a per-(feature, key lane) value; valid for tid < D.
    auto feature_sum = [&](double x) {
        __syncthreads();
        part[tid] = x;
        __syncthreads();
        double s = 0.0;
        if (tid < D)
            for (int l = 0; l < KL; ++l) s += part[l * D + tid];
        return s;
    };
    // Stage keys [c0, c0 + nk) (values too if asked), rows past the prefix zero.
    auto load_chunk = [&](int c0, int nk, bool with_v) {
        for (int e = tid; e < CHK * D; e += NT) {
            const int jj = e / D, a = e % D;
            double kk = 0.0, vv = 0.0;
            if (jj < nk) {
                const int64_t off = static_cast<int64_t>(c0 + jj) * D + a;
                kk = load_f64(kh, off);
                if (with_v) vv = load_f64(vh, off);
            }
            Ks[jj * LD + a] = kk;
            if (with_v) Vs[jj * LD + a] = vv;
        }
    };
    // Dot product of the staged key tid / G with `vec` (minus `shift` if given), valid in every
    // lane of the group.
    auto key_dot = [&](const double* vec, const double* shift) -> double {
        const int jj = tid / G, g = tid % G;
        double s = 0.0;
#pragma unroll
        for (int t = 0; t < DG; ++t) {
            const int a = g * DG + t;
            s += vec[a] * (shift ? Ks[jj * LD + a] - shift[a] : Ks[jj * LD + a]);
        }
#pragma unroll
        for (int off = G / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, G);
        return s;
    };
    __syncthreads();

    // ---- pass 0: row maximum
    double mloc = -INFINITY;
    for (int c0 = 0; c0 < cnt; c0 += CHK) {
        const int nk = min(CHK, cnt - c0);
        load_chunk(c0, nk, false);
        __syncthreads();
        const double s = key_dot(qs, nullptr) * inv_h;
        if (tid / G < nk) mloc = fmax(mloc, s);
        __syncthreads();
    }
    const double m = block_sum(mloc, true);

    // ---- pass 1: omega, kbar, vbar
    double aw = 0.0, ak = 0.0, av = 0.0;
    for (int c0 = 0; c0 < cnt; c0 += CHK) {
        const int nk = min(CHK, cnt - c0);
        load_chunk(c0, nk, true);
        __syncthreads();
        const double s = key_dot(qs, nullptr) * inv_h;
        if (tid % G == 0) ws[tid / G] = tid / G < nk ? exp(s - m) : 0.0;
        __syncthreads();
        for (int jj = kl; jj < nk; jj += KL) {
            ak += ws[jj] * Ks[jj * LD + fa];
            av += ws[jj] * Vs[jj * LD + fa];
        }
        if (tid < nk) aw += ws[tid];
        __syncthreads();
    }
    const double omega = block_sum(aw, false);
    const double skb = feature_sum(ak);
    const double svb = feature_sum(av);
    if (tid < D) {
        kbar[tid] = skb / omega;
        vbar[tid] = svb / omega;
    }
    __syncthreads();

    // ---- CG on A x = kbar - q (thread tid < D holds x, r, p of feature tid; p also in LDS)
    const double ridge = lambda * exp(-m);
    double xr = 0.0, rr_ = 0.0, pr = 0.0;
    if (tid < D) {
        rr_ = kbar[tid] - qs[tid];
        pr = rr_;
        ps[tid] = pr;
        xs[tid] = 0.0;
    }
    double rho = block_sum(tid < D ? rr_ * rr_ : 0.0, false);
    const double stop = tol * tol * rho;
    for (int it = 0; it < max_iter && rho > stop; ++it) {
        __syncthreads();   // ps published
        double acc = 0.0;
        for (int c0 = 0; c0 < cnt; c0 += CHK) {
            const int nk = min(CHK, cnt - c0);
            load_chunk(c0, nk, false);
            __syncthreads();
            const double s = key_dot(qs, nullptr) * inv_h;
            const double u = key_dot(ps, kbar);
            if (tid % G == 0) ws[tid / G] = tid / G < nk ? exp(s - m) * u : 0.0;
            __syncthreads();
            for (int jj = kl; jj < nk; jj += KL) acc += ws[jj] * (Ks[jj * LD + fa] - kbar[fa]);
            __syncthreads();
        }
        double ap = feature_sum(acc);
        if (tid < D) ap += ridge * pr;
        const double pap = block_sum(tid < D ? pr * ap : 0.0, false);
        if (!(pap > 0.0)) break;   // uniform: every thread holds the same sum
        const double alpha = rho / pap;
        if (tid < D) {
            xr += alpha * pr;
            rr_ -= alpha * ap;
        }
        const double rho_new = block_sum(tid < D ? rr_ * rr_ : 0.0, false);
        const double beta = rho_new / rho;
        rho = rho_new;
        if (tid < D) {
            pr = rr_ + beta * pr;
            ps[tid] = pr;
        }
    }
    const bool converged = rho <= stop;   // uniform
    if (!converged) {   // the direct solve takes the row
        if (tid == 0) list[atomicAdd(count, 1u)] = bh * n + i;
        return;
    }
    __syncthreads();
    if (tid < D) xs[tid] = xr;
    __syncthreads();

    // ---- output b = vbar - sum_j wt_j ((k_j - kbar) . x)(v_j - vbar)
    double ao = 0.0;
    for (int c0 = 0; c0 < cnt; c0 += CHK) {
        const int nk = min(CHK, cnt - c0);
        load_chunk(c0, nk, true);
        __syncthreads();
        const double s = key_dot(qs, nullptr) * inv_h;
        const double u = key_dot(xs, kbar);
        if (tid % G == 0) ws[tid / G] = tid / G < nk ? exp(s - m) * u : 0.0;
        __syncthreads();
        for (int jj = kl; jj < nk; jj += KL) ao += ws[jj] * (Vs[jj * LD + fa] - vbar[fa]);
        __syncthreads();
    }
    const double so = feature_sum(ao);
    if (tid < D) out[base + static_cast<int64_t>(i) * D + tid] = static_cast<float>(vbar[tid] - so);
}

// The count of rows handed to the direct solve starts at zero (a kernel, not a memset, so
// that the sequence can be captured in a graph).
__global__ void lla_cg_clear_kernel(unsigned* __restrict__ count) { *count = 0u; }

template <typename TIn, int D>
hipError_t launch_cg_t(const Problem& p, unsigned* count, int* list) {
    const int BH = static_cast<int>(p.B * p.H);
    const unsigned blocks = static_cast<unsigned>(p.B * p.H * p.n);
    lla_cg_clear_kernel<<<dim3(1), dim3(1), 0, p.stream>>>(count);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    prof_begin(p.stream, "lla_cg_kernel");
    lla_cg_kernel<TIn, D><<<dim3(blocks), dim3(CG_NT), 0, p.stream>>>(
        static_cast<const TIn*>(p.q), static_cast<const TIn*>(p.k), static_cast<const TIn*>(p.v), p.out,
        static_cast<int>(p.n), BH, 1.0 / p.h, p.lambda, kCgMaxIterFactor * static_cast<int>(p.d), kCgTol, count,
        list);
    prof_end(p.stream);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const int64_t rows = p.B * p.H * p.n;
    return launch_exact_list(p, list, reinterpret_cast<const int*>(count), static_cast<int>(rows < 2048 ? rows : 2048));
}

template <typename TIn>
hipError_t launch_cg_d(const Problem& p, unsigned* count, int* list) {
    switch (p.d) {
        case 16: return launch_cg_t<TIn, 16>(p, count, list);
        case 32: return launch_cg_t<TIn, 32>(p, count, list);
        case 64: return launch_cg_t<TIn, 64>(p, count, list);
        case 128: return launch_cg_t<TIn, 128>(p, count, list);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t cg_workspace_bytes(int64_t B, int64_t H, int64_t n) {
    return 256 + ((static_cast<size_t>(B * H * n) * 4 + 255) & ~size_t(255));
}

hipError_t launch_cg(const Problem& p, void* workspace) {
    auto* count = static_cast<unsigned*>(workspace);
    auto* list = reinterpret_cast<int*>(static_cast<unsigned char*>(workspace) + 256);
    return p.dtype == 0 ? launch_cg_d<float>(p, count, list) : launch_cg_d<uint16_t>(p, count, list);
}

}  // namespace lla
