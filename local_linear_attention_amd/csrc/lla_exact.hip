// fp64-accumulating causal LLA forward: one workgroup per query row.
//
// Every step follows the centred closed form of the LLA intercept (the "Parallax" blog
// post, section 2 "Canonical Formulation" for the estimator and its moments, Appendix E
// "Boundary amplification is non-negative" for the rank-one split that yields the
// centred form), with the safe-softmax per-row shift of the arXiv page's scoring-form
// paragraph applied to both the weights and the ridge:
//
//   pass 0   m     = max_j q.k_j / h                               (j <= i)
//   pass 1   omega = sum_j wt_j, kbar = sum wt k / omega, vbar = sum wt v / omega,
//            wt_j  = exp(q.k_j / h - m)
//   pass 2   A     = sum_j wt_j (k_j - kbar)(k_j - kbar)^T + lambda e^{-m} I
//            R     = sum_j wt_j (k_j - kbar)(v_j - vbar)^T           (= C_vk^T)
//   solve    Cholesky elimination of [A | kbar - q | R]: the right-hand sides come out as
//            u = L^{-1}(kbar - q) and G = L^{-1} R, so that
//            b = vbar - G^T u = vbar - C_vk A^{-1} (kbar - q) with no back substitution.
//
// Everything after the load is fp64, so the path meets fp32-input accuracy on
// ill-conditioned rows (small lambda e^{-m}, prefixes shorter than d).  It serves every
// (dtype, d) the library accepts and is the reference-grade path for fp32 inputs.
//
// Thread layout: a TR x TC grid; thread (tr, tc) owns rows a = tr + TR*r (r < D/TR) and
// columns b = tc + TC*c (c < D/TC) of A and R in registers.  K/V chunks are staged in
// LDS; the solve broadcasts one pivot column and one right-hand-side row per step.
#include "lla_device.h"
#include "lla_internal.h"

#include <math.h>

namespace lla {
namespace {

template <int D> struct ExactCfg;
template <> struct ExactCfg<16> { static constexpr int TR = 16, TC = 16; };
template <> struct ExactCfg<32> { static constexpr int TR = 16, TC = 16; };
template <> struct ExactCfg<64> { static constexpr int TR = 16, TC = 16; };
template <> struct ExactCfg<128> { static constexpr int TR = 16, TC = 32; };

// LIST = false: block b computes row rows - 1 - b / BH of head b % BH (rows 0 .. rows-1 of
// every head, longest first).  LIST = true: the blocks share the *count rows listed in
// `list` (entry bh * n + i), block b taking entries b, b + gridDim.x, ... -- the rows the
// matrix-core path hands back (see the guard of lla_fast.hip).
template <typename TIn, int D, bool LIST>
__global__ __launch_bounds__(ExactCfg<D>::TR * ExactCfg<D>::TC)
void lla_exact_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                      const TIn* __restrict__ v, float* __restrict__ out,
                      int n, int rows, int BH, double inv_h, double lambda,
                      const int* __restrict__ list, const int* __restrict__ count) {
    constexpr int TR = ExactCfg<D>::TR, TC = ExactCfg<D>::TC, NT = TR * TC;
    constexpr int RA = D / TR, CB = D / TC;
    constexpr int CHK = 2048 / D;   // keys per staged chunk (16 KiB of fp64 per array)
    constexpr int G = NT / CHK;     // threads per key in the score dot product
    constexpr int DG = D / G;       // features per thread in the score dot product
    constexpr int KL = NT / D;      // key lanes in the first-moment pass
    constexpr int LD = D + 1;       // padded LDS row
    static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "score group must be a power of 2");
    static_assert(D % G == 0 && NT % D == 0 && D % TR == 0 && D % TC == 0, "layout");

    __shared__ double qs[D];
    __shared__ double Ks[CHK * LD];
    __shared__ double Vs[CHK * LD];
    __shared__ double ws[CHK];
    __shared__ double kbar[D], vbar[D];
    __shared__ double red[NT];
    __shared__ double colp[D], rowp[D], zs[D], us[D];
    __shared__ double part[TR * D];

    const int tid = threadIdx.x;
    const int tr = tid / TC, tc = tid % TC;
    auto row_body = [&](const int i, const int bh) {
    const int64_t base = static_cast<int64_t>(bh) * n * D;
    const TIn* kh = k + base;
    const TIn* vh = v + base;
    const int cnt = i + 1;

    for (int e = tid; e < D; e += NT) qs[e] = load_f64(q + base, static_cast<int64_t>(i) * D + e);

    // Stage keys [c0, c0 + nk) (and values) as fp64; rows past the prefix are zero.
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
    // Score of key tid/G of the staged chunk (valid in every lane of the group).
    auto chunk_score = [&]() -> double {
        const int jj = tid / G, g = tid % G;
        double s = 0.0;
#pragma unroll
        for (int t = 0; t < DG; ++t) s += qs[g * DG + t] * Ks[jj * LD + g * DG + t];
#pragma unroll
        for (int off = G / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, G);
        return s * inv_h;
    };

    __syncthreads();

    // ---- pass 0: row maximum of the scores
    double mloc = -INFINITY;
    for (int c0 = 0; c0 < cnt; c0 += CHK) {
        const int nk = min(CHK, cnt - c0);
        load_chunk(c0, nk, false);
        __syncthreads();
        const double s = chunk_score();
        if (tid / G < nk) mloc = fmax(mloc, s);
        __syncthreads();
    }
    red[tid] = mloc;
    __syncthreads();
    for (int s = NT / 2; s > 0; s >>= 1) {
        if (tid < s) red[tid] = fmax(red[tid], red[tid + s]);
        __syncthreads();
    }
    const double m = red[0];
    __syncthreads();

    // ---- pass 1: omega, weighted key and value means
    const int fa = tid % D, kl = tid / D;
    double acc_w = 0.0, acc_k = 0.0, acc_v = 0.0;
    for (int c0 = 0; c0 < cnt; c0 += CHK) {
        const int nk = min(CHK, cnt - c0);
        load_chunk(c0, nk, true);
        __syncthreads();
        const double s = chunk_score();
        if (tid % G == 0) ws[tid / G] = (tid / G < nk) ? exp(s - m) : 0.0;
        __syncthreads();
        for (int jj = kl; jj < nk; jj += KL) {
            const double w = ws[jj];
            acc_w += w;
            acc_k += w * Ks[jj * LD + fa];
            acc_v += w * Vs[jj * LD + fa];
        }
        __syncthreads();
    }
    part[kl * D + fa] = acc_k;
    if (fa == 0) red[kl] = acc_w;
    __syncthreads();
    double sk = 0.0, omega = 0.0;
    if (tid < D) {
        for (int t = 0; t < KL; ++t) { sk += part[t * D + tid]; omega += red[t]; }
    }
    __syncthreads();
    part[kl * D + fa] = acc_v;
    __syncthreads();
    if (tid < D) {
        double sv = 0.0;
        for (int t = 0; t < KL; ++t) sv += part[t * D + tid];
        kbar[tid] = sk / omega;
        vbar[tid] = sv / omega;
    }
    __syncthreads();

    // ---- pass 2: centred second moments A = C_kk, R = C_vk^T
    double A[RA][CB], R[RA][CB];
#pragma unroll
    for (int r = 0; r < RA; ++r)
#pragma unroll
        for (int c = 0; c < CB; ++c) { A[r][c] = 0.0; R[r][c] = 0.0; }

    for (int c0 = 0; c0 < cnt; c0 += CHK) {
        const int nk = min(CHK, cnt - c0);
        load_chunk(c0, nk, true);
        __syncthreads();
        const double s = chunk_score();
        if (tid % G == 0) ws[tid / G] = (tid / G < nk) ? exp(s - m) : 0.0;
        __syncthreads();  // scores read the raw keys before they are centred in place
        for (int e = tid; e < nk * D; e += NT) {
            const int jj = e / D, a = e % D;
            Ks[jj * LD + a] -= kbar[a];
            Vs[jj * LD + a] -= vbar[a];
        }
        __syncthreads();
        for (int jj = 0; jj < nk; ++jj) {
            const double w = ws[jj];
            double ka[RA], kb[CB], vb[CB];
#pragma unroll
            for (int r = 0; r < RA; ++r) ka[r] = w * Ks[jj * LD + tr + TR * r];
#pragma unroll
            for (int c = 0; c < CB; ++c) {
                kb[c] = Ks[jj * LD + tc + TC * c];
                vb[c] = Vs[jj * LD + tc + TC * c];
            }
#pragma unroll
            for (int r = 0; r < RA; ++r)
#pragma unroll
                for (int c = 0; c < CB; ++c) {
                    A[r][c] = fma(ka[r], kb[c], A[r][c]);
                    R[r][c] = fma(ka[r], vb[c], R[r][c]);
                }
        }
        __syncthreads();
    }

    // ---- ridge (rescaled by the same shift as the weights) and right-hand side
    const double lam_s = lambda * exp(-m);
    double dmax = 0.0;
#pragma unroll
    for (int r = 0; r < RA; ++r)
#pragma unroll
        for (int c = 0; c < CB; ++c)
            if (tr + TR * r == tc + TC * c) {
                A[r][c] += lam_s;
                dmax = fmax(dmax, A[r][c]);
            }
    red[tid] = dmax;
    if (tid < D) zs[tid] = kbar[tid] - qs[tid];
    __syncthreads();
    for (int s = NT / 2; s > 0; s >>= 1) {
        if (tid < s) red[tid] = fmax(red[tid], red[tid + s]);
        __syncthreads();
    }
    // lambda > 0: the matrix is positive definite, only non-positive pivots (possible
    // only through rounding) are dropped.  lambda = 0: pivots below 1e-12 of the largest
    // diagonal mark a direction the prefix does not determine and are dropped.
    const double thresh = (lambda > 0.0) ? 0.0 : 1e-12 * red[0];

    // ---- Cholesky elimination of [A | z | R]
    for (int p = 0; p < D; ++p) {
        const int pcc = p / TC, prr = p / TR;
        if (tc == p % TC) {
#pragma unroll
            for (int r = 0; r < RA; ++r)
#pragma unroll
                for (int c = 0; c < CB; ++c)
                    if (c == pcc) colp[tr + TR * r] = A[r][c];
        }
        if (tr == p % TR) {
#pragma unroll
            for (int r = 0; r < RA; ++r)
                if (r == prr) {
#pragma unroll
                    for (int c = 0; c < CB; ++c) rowp[tc + TC * c] = R[r][c];
                }
        }
        __syncthreads();
        const double piv = colp[p];
        const double inv = (piv > thresh) ? 1.0 / sqrt(piv) : 0.0;
        const double up = zs[p] * inv;
#pragma unroll
        for (int r = 0; r < RA; ++r) {
            const int a = tr + TR * r;
            if (a > p) {
                const double lap = colp[a] * inv;
#pragma unroll
                for (int c = 0; c < CB; ++c) {
                    const int b = tc + TC * c;
                    if (b > p) A[r][c] = fma(-lap, colp[b] * inv, A[r][c]);
                    R[r][c] = fma(-lap, rowp[b] * inv, R[r][c]);
                }
                if (tc == 0) zs[a] = fma(-lap, up, zs[a]);
            } else if (a == p) {
#pragma unroll
                for (int c = 0; c < CB; ++c) R[r][c] *= inv;
            }
        }
        if (tid == 0) us[p] = up;
        __syncthreads();
    }

    // ---- b = vbar - G^T u
#pragma unroll
    for (int c = 0; c < CB; ++c) {
        double acc = 0.0;
#pragma unroll
        for (int r = 0; r < RA; ++r) acc = fma(R[r][c], us[tr + TR * r], acc);
        part[tr * D + tc + TC * c] = acc;
    }
    __syncthreads();
    if (tid < D) {
        double acc = 0.0;
        for (int t = 0; t < TR; ++t) acc += part[t * D + tid];
        out[base + static_cast<int64_t>(i) * D + tid] = static_cast<float>(vbar[tid] - acc);
    }
    };
    if constexpr (!LIST) {
        row_body(rows - 1 - static_cast<int>(blockIdx.x / BH), static_cast<int>(blockIdx.x % BH));
    } else {
        const int cnt = *count;
        for (int e = static_cast<int>(blockIdx.x); e < cnt; e += static_cast<int>(gridDim.x)) {
            const int code = list[e];
            row_body(code % n, code / n);
            __syncthreads();   // the next row restages every shared array
        }
    }
}

template <typename TIn, int D>
hipError_t launch_exact_t(const Problem& p, int rows) {
    constexpr int NT = ExactCfg<D>::TR * ExactCfg<D>::TC;
    const int BH = static_cast<int>(p.B * p.H);
    const unsigned blocks = static_cast<unsigned>(p.B * p.H * rows);
    prof_begin(p.stream, "lla_exact_kernel");
    lla_exact_kernel<TIn, D, false><<<dim3(blocks), dim3(NT), 0, p.stream>>>(
        static_cast<const TIn*>(p.q), static_cast<const TIn*>(p.k), static_cast<const TIn*>(p.v),
        p.out, static_cast<int>(p.n), rows, BH, 1.0 / p.h, p.lambda, nullptr, nullptr);
    prof_end(p.stream);
    return hipGetLastError();
}

template <typename TIn, int D>
hipError_t launch_exact_list_t(const Problem& p, const int* list, const int* count, int blocks) {
    constexpr int NT = ExactCfg<D>::TR * ExactCfg<D>::TC;
    const int BH = static_cast<int>(p.B * p.H);
    prof_begin(p.stream, "lla_exact_list_kernel");
    lla_exact_kernel<TIn, D, true><<<dim3(static_cast<unsigned>(blocks)), dim3(NT), 0, p.stream>>>(
        static_cast<const TIn*>(p.q), static_cast<const TIn*>(p.k), static_cast<const TIn*>(p.v),
        p.out, static_cast<int>(p.n), 0, BH, 1.0 / p.h, p.lambda, list, count);
    prof_end(p.stream);
    return hipGetLastError();
}

template <typename TIn>
hipError_t launch_exact_list_d(const Problem& p, const int* list, const int* count, int blocks) {
    switch (p.d) {
        case 16: return launch_exact_list_t<TIn, 16>(p, list, count, blocks);
        case 32: return launch_exact_list_t<TIn, 32>(p, list, count, blocks);
        case 64: return launch_exact_list_t<TIn, 64>(p, list, count, blocks);
        case 128: return launch_exact_list_t<TIn, 128>(p, list, count, blocks);
        default: return hipErrorInvalidValue;
    }
}

template <typename TIn>
hipError_t launch_exact_d(const Problem& p, int rows) {
    switch (p.d) {
        case 16: return launch_exact_t<TIn, 16>(p, rows);
        case 32: return launch_exact_t<TIn, 32>(p, rows);
        case 64: return launch_exact_t<TIn, 64>(p, rows);
        case 128: return launch_exact_t<TIn, 128>(p, rows);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_exact(const Problem& p, int rows) {
    if (rows <= 0) return hipSuccess;
    return p.dtype == 0 ? launch_exact_d<float>(p, rows) : launch_exact_d<uint16_t>(p, rows);
}

hipError_t launch_exact_list(const Problem& p, const int* list, const int* count, int blocks) {
    if (blocks <= 0) return hipSuccess;
    return p.dtype == 0 ? launch_exact_list_d<float>(p, list, count, blocks)
                        : launch_exact_list_d<uint16_t>(p, list, count, blocks);
}

}  // namespace lla
