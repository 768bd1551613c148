// Matrix-core path of the causal LLA forward for bf16 inputs, head dimension 64.
//
// Work split (rows are query positions i of one head):
//   * rows i < 2d run on the fp64 kernel: their prefixes hold at most 2d keys, so C_kk is
//     rank-deficient or barely full rank and the ridge lambda e^{-m} alone conditions the
//     solve -- the normal-equation form then needs more than fp16/fp32 precision;
//   * rows i >= 2d run here, in two kernels:
//       lla_stats_kernel    score pass with a running max (FlashAttention-style online
//                           softmax): m_i, omega_i, kbar_i, vbar_i -> workspace;
//       lla_moments_kernel  per query, the centred weighted second moments
//                           C_kk = R_k^T R_k and C_vk^T = R_k^T R_v with
//                           R_k[j] = sqrt(wt_ij) (k_j - kbar_i), R_v[j] = sqrt(wt_ij) (v_j - vbar_i)
//                           rounded once to fp16 (the same rounded R_k on both sides keeps the
//                           two moments consistent), accumulated in fp32 by MFMA; then the
//                           ridge-rescaled SPD solve (C_kk + lambda e^{-m} I) y = kbar - q by
//                           LDL^T elimination in one wave, and b = vbar - C_vk y.
// The estimator, its moments and the centred form follow the "Parallax" blog post, section 2
// "Canonical Formulation" and Appendix E; the max shift is the safe softmax of the arXiv
// page's scoring-form paragraph, with the ridge scaled by the same e^{-m}.
//
// MFMA: v_mfma_f32_16x16x32_{bf16,f16}.  Lane l supplies row/column (l % 16) of A/B and 8
// consecutive K-slots (l / 16); D[4 (l/16) + r][l % 16] lands in accumulator register r.
// Any permutation of the K-slots that A and B share leaves the product unchanged, which the
// stats kernel uses to feed the score tile straight back as the P operand.
#include "lla_internal.h"

#include <math.h>

#include <mutex>

namespace lla {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int FD = 64;              // head dimension of this path
constexpr int SROW = 2 * FD + 4;    // workspace row: kbar[FD], vbar[FD], m, omega, 2 pad
constexpr int KT = 32;              // keys per tile
constexpr int KK_LD = FD + 8;       // key-major bf16 tile row (elements), 144 B
constexpr int XA_LD = KT + 4;       // feature-major f16 row in the stats kernel, 72 B
constexpr int XB_LD = KT + 8;       // feature-major f16 row in the moments kernel, 80 B
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

constexpr int A_WAVES = 4, A_QW = 16, A_QB = A_WAVES * A_QW;  // stats: 64 queries / block
constexpr int B_WAVES = 4;                                     // moments: 1 query per wave

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ float4v mfma_bf16(bf16x8 a, bf16x8 b, float4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float4v mfma_f16(half8 a, half8 b, float4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Stage one tile of KT keys: 256 threads, thread -> key jj = tid / 8, features f0..f0+7.
// Keys at or past n are zero.  kk (if non-null) receives the bf16 keys key-major; kt and vt
// receive keys and values feature-major as fp16 (exact for bf16 values in fp16 range).
template <int XLD>
__device__ __forceinline__ void stage_tile(const uint16_t* __restrict__ kh,
                                           const uint16_t* __restrict__ vh, int n, int j0,
                                           uint16_t* kk, _Float16* kt, _Float16* vt) {
    const int tid = threadIdx.x;
    const int jj = tid >> 3, f0 = (tid & 7) * 8;
    const int j = j0 + jj;
    uint4 kr = make_uint4(0, 0, 0, 0), vr = make_uint4(0, 0, 0, 0);
    if (j < n) {
        kr = *reinterpret_cast<const uint4*>(kh + static_cast<int64_t>(j) * FD + f0);
        vr = *reinterpret_cast<const uint4*>(vh + static_cast<int64_t>(j) * FD + f0);
    }
    if (kk) *reinterpret_cast<uint4*>(kk + jj * KK_LD + f0) = kr;
    const uint32_t kw[4] = {kr.x, kr.y, kr.z, kr.w};
    const uint32_t vw[4] = {vr.x, vr.y, vr.z, vr.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t kb = (kw[e >> 1] >> (16 * (e & 1))) & 0xffffu;
        const uint32_t vb = (vw[e >> 1] >> (16 * (e & 1))) & 0xffffu;
        kt[(f0 + e) * XLD + jj] = static_cast<_Float16>(bf16_bits_to_f32(kb));
        vt[(f0 + e) * XLD + jj] = static_cast<_Float16>(bf16_bits_to_f32(vb));
    }
}

// ---------------------------------------------------------------------------------------
// Score pass: per query, running max m, omega = sum exp(s - m), kbar, vbar.
// Block = 4 waves x 16 queries; tiles of 32 keys shared through LDS.
__global__ __launch_bounds__(256) void lla_stats_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, float* __restrict__ stats, int n, int row0, int BH,
    float sl2) {
    __shared__ __attribute__((aligned(16))) uint16_t Kk[KT * KK_LD];
    __shared__ __attribute__((aligned(16))) _Float16 Xt[2 * FD * XA_LD];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int nrows = n - row0;
    const int nblk = (nrows + A_QB - 1) / A_QB;
    const int blk = nblk - 1 - static_cast<int>(blockIdx.x / BH);  // longest rows first
    const int bh = static_cast<int>(blockIdx.x % BH);
    const int q0 = row0 + blk * A_QB;
    const int qlast = min(q0 + A_QB, n) - 1;
    const int64_t base = static_cast<int64_t>(bh) * n * FD;
    const uint16_t* kh = k + base;
    const uint16_t* vh = v + base;

    const int qi = q0 + w * A_QW + c;     // this lane's query (column c)
    const int qc = min(qi, n - 1);
    const int wave_last = min(q0 + w * A_QW + A_QW - 1, n - 1);
    bf16x8 qf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
        qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(
                                                q + base + static_cast<int64_t>(qc) * FD + ks * 32 + 8 * g));

    float m_run = -INFINITY, l_run = 0.0f;
    float4v o[8];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) o[mb] = float4v{0.f, 0.f, 0.f, 0.f};

    const int ntiles = (qlast + KT) / KT;
    for (int t = 0; t < ntiles; ++t) {
        const int j0 = t * KT;
        __syncthreads();
        stage_tile<XA_LD>(kh, vh, n, j0, Kk, Xt, Xt + FD * XA_LD);
        __syncthreads();
        if (j0 > wave_last) continue;  // wave-uniform: no key of this tile is in any prefix

        // S^T blocks: lane holds keys j0 + kb*16 + 4g + r for query qi.
        float x[8];
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            float4v s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 a = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const uint4*>(Kk + (kb * 16 + c) * KK_LD + ks * 32 + 8 * g));
                s = mfma_bf16(a, qf[ks], s);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = j0 + kb * 16 + 4 * g + r;
                const float val = (j <= qc) ? s[r] * sl2 : -INFINITY;
                x[kb * 4 + r] = val;
                tmax = fmaxf(tmax, val);
            }
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m_run, tmax);   // finite: key 0 is in every prefix
        const float alpha = exp2f(m_run - m_new);
        float psum = 0.0f;
        half8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float pe = exp2f(x[e] - m_new);
            psum += pe;
            pb[e] = static_cast<_Float16>(pe);
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
        // O^T[f][query] += X^T[f][keys] P^T[keys][query], K-slots = keys {4g..4g+3, 16+4g..}.
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
            o[mb] *= alpha;
            const _Float16* row = Xt + (mb * 16 + c) * XA_LD;
            const half4 lo = *reinterpret_cast<const half4*>(row + 4 * g);
            const half4 hi = *reinterpret_cast<const half4*>(row + 16 + 4 * g);
            const half8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            o[mb] = mfma_f16(a, pb, o[mb]);
        }
    }
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (qi < n) {
        float* srow = stats + (static_cast<int64_t>(bh) * nrows + (qi - row0)) * SROW;
        const float inv = 1.0f / l_tot;
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
            *reinterpret_cast<float4v*>(srow + mb * 16 + 4 * g) = o[mb] * inv;
        if (g == 0) {
            srow[2 * FD] = m_run * LN2;   // back to natural units of q.k/h
            srow[2 * FD + 1] = l_tot;
        }
    }
}

// ---------------------------------------------------------------------------------------
// Moments + solve: block = 4 waves, one query per wave (4 consecutive rows of one head).
constexpr int B_TILE_BYTES = KT * KK_LD * 2 + 2 * FD * XB_LD * 2 + B_WAVES * KT * 2;
constexpr int B_SOLVE_FLOATS = FD * (FD + 1) + 2 * FD;  // A (padded rows) + pivot column + y
constexpr int B_SMEM = (B_SOLVE_FLOATS * 4 * B_WAVES > B_TILE_BYTES) ? B_SOLVE_FLOATS * 4 * B_WAVES
                                                                       : B_TILE_BYTES;

__global__ __launch_bounds__(256) void lla_moments_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ stats, float* __restrict__ out,
    int n, int row0, int BH, float sl2, float lambda) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint16_t* Kk = reinterpret_cast<uint16_t*>(smem);
    _Float16* Kt = reinterpret_cast<_Float16*>(smem + KT * KK_LD * 2);
    _Float16* Vt = Kt + FD * XB_LD;
    _Float16* Sw = Vt + FD * XB_LD;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int nrows = n - row0;
    const int nblk = (nrows + B_WAVES - 1) / B_WAVES;
    const int blk = nblk - 1 - static_cast<int>(blockIdx.x / BH);  // longest rows first
    const int bh = static_cast<int>(blockIdx.x % BH);
    const int i0 = row0 + blk * B_WAVES;
    const int i = i0 + w;
    const bool valid = i < n;
    const int ic = min(i, n - 1);
    const int last = min(i0 + B_WAVES - 1, n - 1);
    const int64_t base = static_cast<int64_t>(bh) * n * FD;
    const uint16_t* kh = k + base;
    const uint16_t* vh = v + base;
    const float* st = stats + (static_cast<int64_t>(bh) * nrows + (ic - row0)) * SROW;

    // Centring constants of this wave's query, rounded to fp16, for feature c + 16 fb.
    half8 nkb[4], nvb[4];
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) {
        const _Float16 kb = static_cast<_Float16>(-st[fb * 16 + c]);
        const _Float16 vb = static_cast<_Float16>(-st[FD + fb * 16 + c]);
#pragma unroll
        for (int e = 0; e < 8; ++e) { nkb[fb][e] = kb; nvb[fb][e] = vb; }
    }
    // Score operands of waves 0 and 1: column c < B_WAVES is query i0 + c.
    const int qcol = min(i0 + c, n - 1);
    const bool colv = c < B_WAVES;
    const float mcol = stats[(static_cast<int64_t>(bh) * nrows + (qcol - row0)) * SROW + 2 * FD] * LOG2E;
    bf16x8 qf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (colv) raw = *reinterpret_cast<const uint4*>(q + base + static_cast<int64_t>(qcol) * FD + ks * 32 + 8 * g);
        qf[ks] = __builtin_bit_cast(bf16x8, raw);
    }

    float4v ckk[10], cvk[16];
#pragma unroll
    for (int t = 0; t < 10; ++t) ckk[t] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 16; ++t) cvk[t] = float4v{0.f, 0.f, 0.f, 0.f};

    const int ntiles = (last + KT) / KT;
    for (int t = 0; t < ntiles; ++t) {
        const int j0 = t * KT;
        __syncthreads();
        stage_tile<XB_LD>(kh, vh, n, j0, Kk, Kt, Vt);
        __syncthreads();
        if (w < 2) {
            // sqrt of the shifted weights, exp((s - m)/2), for key block kb = w.
            float4v s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 a = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const uint4*>(Kk + (w * 16 + c) * KK_LD + ks * 32 + 8 * g));
                s = mfma_bf16(a, qf[ks], s);
            }
            if (colv) {
                half4 sw4;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = j0 + w * 16 + 4 * g + r;
                    sw4[r] = static_cast<_Float16>(j <= qcol ? exp2f((s[r] * sl2 - mcol) * 0.5f) : 0.0f);
                }
                *reinterpret_cast<half4*>(Sw + c * KT + w * 16 + 4 * g) = sw4;
            }
        }
        __syncthreads();
        if (j0 > ic) continue;  // wave-uniform: the whole tile lies past this wave's query

        const half8 sw = *reinterpret_cast<const half8*>(Sw + w * KT + 8 * g);
        half8 rk[4], rv[4];
#pragma unroll
        for (int fb = 0; fb < 4; ++fb) {
            const half8 kf = *reinterpret_cast<const half8*>(Kt + (fb * 16 + c) * XB_LD + 8 * g);
            const half8 vf = *reinterpret_cast<const half8*>(Vt + (fb * 16 + c) * XB_LD + 8 * g);
            rk[fb] = (kf + nkb[fb]) * sw;
            rv[fb] = (vf + nvb[fb]) * sw;
        }
        int idx = 0;
#pragma unroll
        for (int fb = 0; fb < 4; ++fb)
#pragma unroll
            for (int fb2 = fb; fb2 < 4; ++fb2) { ckk[idx] = mfma_f16(rk[fb], rk[fb2], ckk[idx]); ++idx; }
#pragma unroll
        for (int fb = 0; fb < 4; ++fb)
#pragma unroll
            for (int fv = 0; fv < 4; ++fv) cvk[fb * 4 + fv] = mfma_f16(rk[fb], rv[fv], cvk[fb * 4 + fv]);
    }
    __syncthreads();  // tile buffers are dead; the solve area aliases them

    // ---- ridge-rescaled SPD solve, lane a owns row a
    constexpr int ALD = FD + 1;
    float* A = reinterpret_cast<float*>(smem) + w * B_SOLVE_FLOATS;
    float* colb = A + FD * ALD;
    float* yv = colb + FD;
    {
        int idx = 0;
#pragma unroll
        for (int fb = 0; fb < 4; ++fb)
#pragma unroll
            for (int fb2 = fb; fb2 < 4; ++fb2) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = fb * 16 + 4 * g + r, col = fb2 * 16 + c;
                    A[row * ALD + col] = ckk[idx][r];
                    if (fb != fb2) A[col * ALD + row] = ckk[idx][r];
                }
                ++idx;
            }
    }
    const float m_x = st[2 * FD] * LOG2E;
    const float lam_s = lambda * exp2f(-m_x);
    A[lane * ALD + lane] += lam_s;
    float dmax = A[lane * ALD + lane];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) dmax = fmaxf(dmax, __shfl_xor(dmax, off));
    // lambda > 0: drop only pivots that rounding made non-positive; lambda = 0: also drop
    // directions the prefix leaves (numerically) undetermined.
    const float thresh = lambda > 0.0f ? 0.0f : 1e-6f * dmax;

    float ar[FD];
#pragma unroll
    for (int b = 0; b < FD; ++b) ar[b] = A[lane * ALD + b];
    const float qa = bf16_bits_to_f32(q[base + static_cast<int64_t>(ic) * FD + lane]);
    float z = st[lane] - qa;

    // Forward elimination (symmetric, no pivoting): after step p, lane p's registers hold row
    // p of U = D L^T and z holds L^{-1} (kbar - q).  Column p of the trailing matrix equals
    // its row p, so one LDS word per lane broadcasts the pivot row.
#pragma unroll
    for (int p = 0; p < FD; ++p) {
        colb[lane] = ar[p];
        const float piv = colb[p];
        const float inv = piv > thresh ? 1.0f / piv : 0.0f;
        const float f = lane > p ? ar[p] * inv : 0.0f;
        const float zp = __shfl(z, p);
        z = fmaf(-f, zp, z);
#pragma unroll
        for (int b = p + 1; b < FD; ++b) ar[b] = fmaf(-f, colb[b], ar[b]);
    }
    // Back substitution U y = z, column by column.
    float ylane = 0.0f;
#pragma unroll
    for (int p = FD - 1; p >= 0; --p) {
        const float dp = __shfl(ar[p], p);
        const float zp = __shfl(z, p);
        const float yp = dp > thresh ? zp / dp : 0.0f;
        ylane = lane == p ? yp : ylane;
        z = fmaf(-ar[p], yp, z);
    }
    yv[lane] = ylane;

    // b = vbar - C_vk y; lane holds C_vk^T[fb*16 + 4g + r][fv*16 + c].
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) {
        const float4v yy = *reinterpret_cast<const float4v*>(yv + fb * 16 + 4 * g);
#pragma unroll
        for (int fv = 0; fv < 4; ++fv)
#pragma unroll
            for (int r = 0; r < 4; ++r) part[fv] = fmaf(cvk[fb * 4 + fv][r], yy[r], part[fv]);
    }
#pragma unroll
    for (int fv = 0; fv < 4; ++fv) {
        part[fv] += __shfl_xor(part[fv], 16);
        part[fv] += __shfl_xor(part[fv], 32);
    }
    if (valid && g == 0) {
        float* orow = out + base + static_cast<int64_t>(i) * FD;
#pragma unroll
        for (int fv = 0; fv < 4; ++fv) orow[fv * 16 + c] = st[FD + fv * 16 + c] - part[fv];
    }
}

int fast_row0(int64_t n, int64_t d) { return static_cast<int>(n < 2 * d ? n : 2 * d); }

}  // namespace

bool fast_supports(int dtype, int64_t d) { return dtype == 1 && d == FD; }

size_t fast_workspace_bytes(int64_t B, int64_t H, int64_t n, int64_t d) {
    const int64_t rows = n - fast_row0(n, d);
    return rows > 0 ? static_cast<size_t>(B * H * rows * SROW) * sizeof(float) : 0;
}

hipError_t launch_fast(const Problem& p, void* workspace) {
    const int row0 = fast_row0(p.n, p.d);
    hipError_t err = launch_exact(p, row0);
    if (err != hipSuccess || p.n <= row0) return err;
    static std::once_flag attr_once;
    static hipError_t attr_err = hipSuccess;
    std::call_once(attr_once, [] {
        attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(&lla_moments_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, B_SMEM);
    });
    if (attr_err != hipSuccess) return attr_err;

    const int n = static_cast<int>(p.n);
    const int BH = static_cast<int>(p.B * p.H);
    const int nrows = n - row0;
    const float sl2 = static_cast<float>(LOG2E / p.h);
    const auto* q = static_cast<const uint16_t*>(p.q);
    const auto* k = static_cast<const uint16_t*>(p.k);
    const auto* v = static_cast<const uint16_t*>(p.v);
    float* stats = static_cast<float*>(workspace);

    const unsigned blocks_a = static_cast<unsigned>(BH) * ((nrows + A_QB - 1) / A_QB);
    prof_begin(p.stream, "lla_stats_kernel");
    lla_stats_kernel<<<dim3(blocks_a), dim3(256), 0, p.stream>>>(q, k, v, stats, n, row0, BH, sl2);
    prof_end(p.stream);
    if ((err = hipGetLastError()) != hipSuccess) return err;

    const unsigned blocks_b = static_cast<unsigned>(BH) * ((nrows + B_WAVES - 1) / B_WAVES);
    prof_begin(p.stream, "lla_moments_kernel");
    lla_moments_kernel<<<dim3(blocks_b), dim3(256), B_SMEM, p.stream>>>(
        q, k, v, stats, p.out, n, row0, BH, sl2, static_cast<float>(p.lambda));
    prof_end(p.stream);
    return hipGetLastError();
}

}  // namespace lla
