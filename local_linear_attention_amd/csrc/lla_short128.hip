// Rows i < 4d of the bf16 d = 128 matrix-core path, in fp64: one workgroup (4 waves) per row.
//
// The row's output is the centred closed form of the LLA intercept ("Parallax" blog post,
// section 2 "Canonical Formulation" for the estimator and its moments, Appendix E for the
// rank-one split behind the centred form), with the safe-softmax shift of the arXiv page's
// scoring-form paragraph applied to the weights and the ridge:
//   w_j = exp(q.k_j / h - m), kbar = sum w k / omega, vbar = sum w v / omega   (j <= i)
//   (C_kk + lambda e^{-m} I) y = kbar - q,   C_kk = sum w (k - kbar)(k - kbar)^T
//   b = vbar - C_vk y = vbar - sum_j w_j u_j (v_j - vbar),   u_j = (k_j - kbar).y
// so the cross moment C_vk is never formed (its product with y is one pass over the values).
//
// Three passes over the prefix, staged through LDS 64 keys at a time (the next chunk's loads
// in flight while the current one is used):
//   1. scores (4 threads per key), their running maximum, and kbar, vbar accumulated on the
//      fly, rescaled when the maximum grows (thread = feature and key parity);
//   2. C_kk on the matrix cores (v_mfma_f64_16x16x4f64, 4 keys per step): the 36 upper 16x16
//      blocks split 9 per wave, R_j = sqrt(w_j) (k_j - kbar) formed per lane;
//   3. after the solve: u_j, then sum_j w_j u_j v_j and sum_j w_j u_j.
// Solve, LDL^T in two 64-row halves, lane per row:
//   phase 1 (64 pivot steps, one barrier each): wave 0 holds rows 0..63 x columns 0..63,
//     wave 1 rows 64..127 x columns 0..63 (its multipliers), waves 2 and 3 rows 64..127 x
//     columns 64..95 and 96..127 (the Schur complement update); column p of rows 0..127 goes
//     through LDS, and by symmetry it is also pivot row p;
//   phase 2: wave 3 gathers the 64 x 64 Schur complement and factors it alone (pivot row
//     exchange through LDS within the wave), then back-substitutes y for rows 64..127;
//   wave 0 subtracts the coupling of rows 0..63 to those unknowns (through the stored
//     multipliers of wave 1) and back-substitutes y for rows 0..63.
// Pivots <= thresh are dropped (their unknowns set to zero): lambda > 0 drops only those that
// rounding made non-positive, lambda = 0 also those below 1e-12 of the largest diagonal entry.
#include "lla_device.h"
#include "lla_internal.h"

#include <math.h>

namespace lla {
namespace {

constexpr int SD = 128;                 // features
constexpr int S8_MAXK = 4 * SD;         // longest prefix: rows i < 4d
constexpr int S8_CH = 64;               // keys per staged chunk
constexpr int S8_KLD = SD + 16;         // bf16 row stride (halves): 72 words, so that the 4 keys
                                        // of an MFMA step fall on distinct bank octets
constexpr int S8_CB = SD + 2;           // one pivot column (128 rows) + the pivot's z (+ pad)
constexpr int S8_ALD = 65;              // fp64 row stride: wave 1's multipliers in transit

// LDS (bytes), sized for two workgroups per CU.  Region M is reused phase by phase:
//   pass 1:   K chunk | V chunk | scores s_j            | partial sums (2 x 128)
//   pass 2:   K chunk |         | sqrt(w_j)
//   transfer: the 36 upper 16x16 blocks of C_kk + ridge (2 KiB each, XOR-swizzled columns)
//   solve:    pivot columns | wave 1's multipliers | phase 2 pivot rows
//   pass 3:   K chunk | V chunk |                      | partial sums
// then the vectors q, kbar, vbar, y, the chunk's w_j u_j, and four reduction slots.
constexpr int S8_KC = 0;
constexpr int S8_VC = S8_KC + S8_CH * S8_KLD * 2;
constexpr int S8_SC = S8_VC + S8_CH * S8_KLD * 2;         // scores, then sqrt(w_j)
constexpr int S8_PART = S8_SC + S8_MAXK * 8;              // 2 x 128 partial sums
constexpr int S8_BLK = 0;                                 // the 36 blocks
constexpr int S8_COL = 0;                                 // two pivot columns (alternating)
constexpr int S8_A21 = 4096;                              // wave 1's rows (after phase 1)
constexpr int S8_XW = S8_A21 + 64 * S8_ALD * 8;           // phase 2 pivot rows, one per wave
constexpr int S8_MSZ = 36 * 256 * 8;
static_assert(S8_PART + 2 * SD * 8 <= S8_MSZ && S8_COL + 2 * S8_CB * 8 <= S8_A21 && S8_XW + 4 * 64 * 8 <= S8_MSZ,
              "the phases' buffers fit in region M");
constexpr int S8_QS = S8_MSZ;                             // q (fp64)
constexpr int S8_KB = S8_QS + SD * 8;                     // kbar
constexpr int S8_VB = S8_KB + SD * 8;                     // vbar
constexpr int S8_YS = S8_VB + SD * 8;                     // y
constexpr int S8_WU = S8_YS + SD * 8;                     // chunk weights, then w_j u_j of a chunk
constexpr int S8_RED = S8_WU + S8_CH * 8;                 // four reduction slots
constexpr int S8_SMEM = S8_RED + 8 * 8;
static_assert(2 * S8_SMEM <= 160 * 1024, "two workgroups per CU");

// Block (I, J), I <= J, of the upper 8 x 8 block triangle, and the LDS double index of its
// entry (m, n): rows of 16, column n stored at n ^ m (conflict-free for row and column reads).
__host__ __device__ constexpr int s8_bidx(int I, int J) { return I * 8 - I * (I - 1) / 2 + (J - I); }
__device__ __forceinline__ int s8_elem(int I, int J, int m, int nn) { return s8_bidx(I, J) * 256 + m * 16 + (nn ^ m); }

// Upper 16x16 blocks (I, J) of C_kk per wave: 9 each, so that waves 0 and 1 need 4 feature
// blocks of R and waves 2 and 3 at most 7.
constexpr int s8_bi[4][9] = {{0, 0, 0, 0, 1, 1, 1, 2, 2},
                             {4, 4, 4, 4, 5, 5, 5, 6, 6},
                             {0, 0, 0, 0, 1, 1, 1, 1, 3},
                             {2, 2, 2, 2, 3, 3, 3, 3, 7}};
constexpr int s8_bj[4][9] = {{0, 1, 2, 3, 1, 2, 3, 2, 3},
                             {4, 5, 6, 7, 5, 6, 7, 6, 7},
                             {4, 5, 6, 7, 4, 5, 6, 7, 3},
                             {4, 5, 6, 7, 4, 5, 6, 7, 7}};
__host__ __device__ constexpr bool s8_uses(int W, int F) {
    for (int b = 0; b < 9; ++b)
        if (s8_bi[W][b] == F || s8_bj[W][b] == F) return true;
    return false;
}

typedef double double4v __attribute__((ext_vector_type(4)));

// The MFMA steps of one staged chunk for wave W (its blocks known at compile time): lane
// (g, c) forms R_j[16 F + c] = sqrt(w_j) (k_j - kbar)[16 F + c] of key j = 4 st + g for the
// feature blocks F its blocks use; A = R of block row I, B = R of block column J.
template <int W>
__device__ __forceinline__ void s8_chunk(double4v (&acc)[9], const uint16_t* __restrict__ kc,
                                         const double* __restrict__ sw, const double (&kbf)[8], int nst,
                                         int g, int c);

// Pins 16 consecutive row entries in registers at this point: the updates that produced them
// are done before it and no LDS load moves across it, which bounds the pivot-row values the
// compiler would otherwise load far ahead of their use (and spill).
#define S8_PIN16(a, o)                                                                              \
    asm volatile("" : "+v"(a[(o) + 0]), "+v"(a[(o) + 1]), "+v"(a[(o) + 2]), "+v"(a[(o) + 3]),     \
                 "+v"(a[(o) + 4]), "+v"(a[(o) + 5]), "+v"(a[(o) + 6]), "+v"(a[(o) + 7]),           \
                 "+v"(a[(o) + 8]), "+v"(a[(o) + 9]), "+v"(a[(o) + 10]), "+v"(a[(o) + 11]),         \
                 "+v"(a[(o) + 12]), "+v"(a[(o) + 13]), "+v"(a[(o) + 14]), "+v"(a[(o) + 15])        \
                 :                                                                                 \
                 : "memory")

// 1 / x from the hardware reciprocal and one Newton step (a pivot's multiplier needs no
// correctly rounded division; the step brings the estimate to full fp64 precision).
__device__ __forceinline__ double s8_rcp(double x) {
    const double r = __builtin_amdgcn_rcp(x);
    return fma(r, fma(-x, r, 1.0), r);
}

__device__ __forceinline__ double bf2d(uint16_t b) { return static_cast<double>(bf16_bits_to_f32(b)); }

__device__ __forceinline__ double wave_max_dd(double x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmax(x, __shfl_xor(x, off));
    return x;
}
__device__ __forceinline__ double wave_sum_dd(double x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

__global__ __launch_bounds__(256, 2) void lla8_short_kernel(const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v,
                                                         float* __restrict__ out, int n, int rows, int BH,
                                                         double inv_h, double lambda) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[S8_SMEM];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c = lane & 15;
    const int i = rows - 1 - static_cast<int>(blockIdx.x) / BH;   // longest rows first
    const int bh = static_cast<int>(blockIdx.x) % BH;
    const int64_t base = static_cast<int64_t>(bh) * n * SD;
    const int nk = i + 1;                                        // keys 0..i
    const int nch = (nk + S8_CH - 1) / S8_CH;

    uint16_t* KC = reinterpret_cast<uint16_t*>(smem + S8_KC);
    uint16_t* VC = reinterpret_cast<uint16_t*>(smem + S8_VC);
    double* QS = reinterpret_cast<double*>(smem + S8_QS);
    double* SC = reinterpret_cast<double*>(smem + S8_SC);
    double* SW = SC;   // sqrt(w_j) replaces the scores after pass 1
    double* PART = reinterpret_cast<double*>(smem + S8_PART);
    double* KB = reinterpret_cast<double*>(smem + S8_KB);
    double* VB = reinterpret_cast<double*>(smem + S8_VB);
    double* YS = reinterpret_cast<double*>(smem + S8_YS);
    double* WU = reinterpret_cast<double*>(smem + S8_WU);
    double* RED = reinterpret_cast<double*>(smem + S8_RED);

    // Chunk staging: thread t copies bytes [64 (t % 4), +64) of key t / 4 of the chunk.
    const int sk = tid >> 2, sq = tid & 3;
    auto fetch = [&](int ch, const uint16_t* src, uint4 (&r)[4]) {
        const int j = ch * S8_CH + sk;
        const uint4* p = reinterpret_cast<const uint4*>(src + base + static_cast<int64_t>(j) * SD + 32 * sq);
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = j < nk ? p[e] : make_uint4(0, 0, 0, 0);
    };
    auto stash = [&](uint16_t* dst, const uint4 (&r)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) *reinterpret_cast<uint4*>(dst + sk * S8_KLD + 32 * sq + 8 * e) = r[e];
    };
    // Block-wide reductions (every thread gets the result).
    auto block_max = [&](double x) {
        x = wave_max_dd(x);
        __syncthreads();
        if (lane == 0) RED[w] = x;
        __syncthreads();
        return fmax(fmax(RED[0], RED[1]), fmax(RED[2], RED[3]));
    };
    auto block_sum = [&](double x) {
        x = wave_sum_dd(x);
        __syncthreads();
        if (lane == 0) RED[w] = x;
        __syncthreads();
        return (RED[0] + RED[1]) + (RED[2] + RED[3]);
    };

    if (tid < SD) QS[tid] = bf2d(q[base + static_cast<int64_t>(i) * SD + tid]);

    // ---- pass 1: scores, running maximum, kbar and vbar (thread = feature f, key parity)
    const int f = tid & (SD - 1), par = tid >> 7;
    double m_run = -INFINITY, ka = 0.0, va = 0.0;
    {
        uint4 rk[4], rv[4];
        fetch(0, k, rk);
        fetch(0, v, rv);
        for (int ch = 0; ch < nch; ++ch) {
            __syncthreads();   // the previous chunk's readers are done
            stash(KC, rk);
            stash(VC, rv);
            if (ch + 1 < nch) {
                fetch(ch + 1, k, rk);
                fetch(ch + 1, v, rv);
            }
            __syncthreads();
            const int j = ch * S8_CH + sk;
            double s = 0.0;
#pragma unroll 8
            for (int e = 0; e < 32; ++e) s = fma(QS[32 * sq + e], bf2d(KC[sk * S8_KLD + 32 * sq + e]), s);
            s += __shfl_xor(s, 1);
            s += __shfl_xor(s, 2);
            s = j < nk ? s * inv_h : -INFINITY;
            if (sq == 0) SC[j] = s;
            const double m_new = fmax(m_run, block_max(s));   // finite: key 0 is in chunk 0
            const double scale = exp(m_run - m_new);
            if (sq == 0) WU[sk] = j < nk ? exp(s - m_new) : 0.0;
            __syncthreads();
            ka *= scale;
            va *= scale;
            for (int kk = par; kk < S8_CH; kk += 2) {
                const double wj = WU[kk];
                ka = fma(wj, bf2d(KC[kk * S8_KLD + f]), ka);
                va = fma(wj, bf2d(VC[kk * S8_KLD + f]), va);
            }
            m_run = m_new;
        }
    }
    const double m = m_run;
    // weights w_j = exp(s_j - m) and sqrt(w_j), zero past the prefix; omega
    double wpart = 0.0;
    for (int j = tid; j < S8_MAXK; j += 256) {
        const double wj = j < nk ? exp(SC[j] - m) : 0.0;
        SW[j] = sqrt(wj);
        wpart += wj;
    }
    const double omega = block_sum(wpart);
    __syncthreads();
    PART[par * SD + f] = ka;
    __syncthreads();
    if (tid < SD) KB[tid] = (PART[tid] + PART[SD + tid]) / omega;
    __syncthreads();
    PART[par * SD + f] = va;
    __syncthreads();
    if (tid < SD) VB[tid] = (PART[tid] + PART[SD + tid]) / omega;
    __syncthreads();

    // ---- pass 2: C_kk, upper blocks (I, J) of this wave, 4 keys per MFMA step
    int bi[9], bj[9];
#pragma unroll
    for (int b = 0; b < 9; ++b) {
        bi[b] = s8_bi[w][b];
        bj[b] = s8_bj[w][b];
    }
    double kbf[8];
#pragma unroll
    for (int F = 0; F < 8; ++F) kbf[F] = KB[16 * F + c];
    double4v acc[9];
#pragma unroll
    for (int b = 0; b < 9; ++b) acc[b] = double4v{0.0, 0.0, 0.0, 0.0};
    {
        uint4 rk[4];
        fetch(0, k, rk);
        for (int ch = 0; ch < nch; ++ch) {
            __syncthreads();
            stash(KC, rk);
            if (ch + 1 < nch) fetch(ch + 1, k, rk);
            __syncthreads();
            const int nst = min(S8_CH, nk - ch * S8_CH + 3) / 4;   // steps holding keys <= i
            const double* swc = SW + ch * S8_CH;
            switch (w) {   // wave-uniform
                case 0: s8_chunk<0>(acc, KC, swc, kbf, nst, g, c); break;
                case 1: s8_chunk<1>(acc, KC, swc, kbf, nst, g, c); break;
                case 2: s8_chunk<2>(acc, KC, swc, kbf, nst, g, c); break;
                default: s8_chunk<3>(acc, KC, swc, kbf, nst, g, c); break;
            }
        }
    }
    // ridge on the diagonal (diagonal blocks: register r of lane (g, c) is row 4r + g, column
    // c), its largest entry
    const double lam_s = lambda * exp(-m);
    double dmax = 0.0;
#pragma unroll
    for (int b = 0; b < 9; ++b) {
        if (bi[b] == bj[b]) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (4 * r + g == c) {
                    acc[b][r] += lam_s;
                    dmax = fmax(dmax, acc[b][r]);
                }
        }
    }
    dmax = block_max(dmax);
    const double thresh = lambda > 0.0 ? 0.0 : 1e-12 * dmax;

    // ---- to lane-per-row form, 16 matrix rows (block row R) per round:
    //   wave 0: rows 0..63 x columns 0..63;  wave 1: rows 64..127 x columns 0..63;
    //   waves 2 and 3: rows 64..127 x columns 64..127 (wave 3 a copy that only keeps pace).
    // The eliminations run as a loop over the four 16-column panels with the 16 pivot steps of
    // a panel unrolled (code that stays in the instruction cache); between panels the row
    // rotates by 16 entries, so that the active panel always sits in cr[0..15] and no
    // register is indexed at run time.  After four panels the row is back in order.
    double* BL = reinterpret_cast<double*>(smem + S8_BLK);
    const int colb = w < 2 ? 0 : 64;                  // first column this wave holds
    const int row = lane + (w == 0 ? 0 : 64);          // its row
    __syncthreads();   // pass 2 done with region M
#pragma unroll
    for (int b = 0; b < 9; ++b) {
        const int I = s8_bi[w][b], J = s8_bj[w][b];
#pragma unroll
        for (int r = 0; r < 4; ++r) BL[s8_elem(I, J, 4 * r + g, c)] = acc[b][r];   // C[16 I + 4r + g][16 J + c]
    }
    __syncthreads();
    double cr[64];
    {
        const int I = row >> 4, m = row & 15;
#pragma unroll
        for (int t = 0; t < 64; ++t) {
            const int J = (colb + t) >> 4, nn = t & 15;   // J wave-uniform
            cr[t] = BL[I <= J ? s8_elem(I, J, m, nn) : s8_elem(J, I, nn, m)];
        }
    }
    auto rotate16 = [&] {   // cr[t] <- cr[(t + 16) % 64]
        double tmp[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) tmp[u] = cr[u];
#pragma unroll
        for (int t = 0; t < 48; ++t) cr[t] = cr[t + 16];
#pragma unroll
        for (int u = 0; u < 16; ++u) cr[48 + u] = tmp[u];
    };
    // right-hand side z = kbar - q of this lane's row
    double z = KB[row] - QS[row];

    // ---- phase 1: pivots 0..63, one code path for every wave.  Waves 0 and 1 publish column
    // p (by symmetry also pivot row p); each wave updates its row's entries in the columns it
    // holds that lie past p (waves 2 and 3: all of them; columns <= p of waves 0 and 1 take a
    // zero multiplier, so that no branch splits the row's registers).  In panel P, entry group
    // G (cr[16 G ..]) holds the original columns of panel (P + G) mod 4.
    double* CB = reinterpret_cast<double*>(smem + S8_COL);
    __syncthreads();   // every row read out of the blocks before the pivot columns overwrite them
    for (int P = 0; P < 4; ++P) {
#pragma unroll
        for (int pp = 0; pp < 16; ++pp) {
            const int p = 16 * P + pp;
            double* cb = CB + (pp & 1) * S8_CB;
            if (w < 2) {
                cb[row] = cr[pp];
                if (row == p) cb[SD] = z;
            }
            __syncthreads();
            const double piv = cb[p];
            const double inv = piv > thresh ? s8_rcp(piv) : 0.0;
            const double fr = row > p ? cb[row] * inv : 0.0;
            z = fma(-fr, cb[SD], z);
            const double frl = colb != 0 ? fr : 0.0;
#pragma unroll
            for (int G = 0; G < 4; ++G) {
                const int panel = (P + G) & 3;
                const double mg = G == 0 ? 0.0 : (P + G <= 3 ? fr : frl);   // group multiplier
                const double* pr = cb + colb + 16 * panel;
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const double mlt = G == 0 ? (u > pp ? fr : frl) : mg;
                    cr[16 * G + u] = fma(-mlt, pr[u], cr[16 * G + u]);
                }
                S8_PIN16(cr, 16 * G);
            }
        }
        rotate16();
    }
    __syncthreads();   // phase 1's column reads done: the staging area is free

    // back substitution of a lane-per-row factor held by one wave (row in order):
    // L^T y = D^{-1} z'
    auto back_sub = [&](double zz) {
        double ylane = 0.0;
        for (int P = 3; P >= 0; --P) {
#pragma unroll
            for (int pp = 15; pp >= 0; --pp) {
                const int p = 16 * P + pp;
                const double cp = P == 3 ? cr[48 + pp] : P == 2 ? cr[32 + pp] : P == 1 ? cr[16 + pp] : cr[pp];
                const double dp = __shfl(cp, p);
                const double zp = __shfl(zz, p);
                const double yp = dp > thresh ? zp * s8_rcp(dp) : 0.0;
                ylane = lane == p ? yp : ylane;
                zz = fma(-cp, yp, zz);
            }
        }
        return ylane;
    };
    double* A21 = reinterpret_cast<double*>(smem + S8_A21);
    if (w == 1) {
        // wave 1's multipliers, for the coupling of rows 0..63 to the unknowns of rows 64..127
#pragma unroll
        for (int t = 0; t < 64; ++t) A21[lane * S8_ALD + t] = cr[t];
    }
    // ---- phase 2: wave 2 factors the 64 x 64 Schur complement, then solves for y of rows
    // 64..127.  Every wave runs the elimination on its own pivot-row buffer, the others with
    // a zero multiplier (their rows unchanged), so that no branch splits the row's registers.
    {
        double* xw = reinterpret_cast<double*>(smem + S8_XW) + 64 * w;
        const bool act = w == 2;
        for (int P = 0; P < 4; ++P) {
#pragma unroll
            for (int pp = 0; pp < 16; ++pp) {
                const int p = 16 * P + pp;
                const double cp = cr[pp];
                xw[lane] = cp;
                LDS_FENCE();
                const double piv = xw[p];
                const double inv = piv > thresh ? s8_rcp(piv) : 0.0;
                const double fr = act && lane > p ? cp * inv : 0.0;
                const double zp = __shfl(z, p);
                z = fma(-fr, zp, z);
#pragma unroll
                for (int G = 0; G < 4; ++G) {
                    const int panel = (P + G) & 3;
                    const double mg = G == 0 ? 0.0 : (P + G <= 3 ? fr : 0.0);
                    const double* pr = xw + 16 * panel;
#pragma unroll
                    for (int u = 0; u < 16; ++u) {
                        const double mlt = G == 0 ? (u > pp ? fr : 0.0) : mg;
                        cr[16 * G + u] = fma(-mlt, pr[u], cr[16 * G + u]);
                    }
                    S8_PIN16(cr, 16 * G);
                }
            }
            rotate16();
        }
    }
    if (w == 2) YS[64 + lane] = back_sub(z);
    __syncthreads();
    if (w == 0) {
        // z_q -= sum_{p >= 64} U[q][p] y_p, U[q][p] = wave 1's entry (row p, column q)
        double s = 0.0;
        for (int pp = 0; pp < 64; ++pp) s = fma(A21[pp * S8_ALD + lane], YS[64 + pp], s);
        YS[lane] = back_sub(z - s);
    }
    __syncthreads();

    // ---- pass 3: u_j = (k_j - kbar).y, then sum_j w_j u_j v_j and sum_j w_j u_j
    double acc_o = 0.0, swu = 0.0;
    {
        uint4 rk[4], rv[4];
        fetch(0, k, rk);
        fetch(0, v, rv);
        for (int ch = 0; ch < nch; ++ch) {
            __syncthreads();
            stash(KC, rk);
            stash(VC, rv);
            if (ch + 1 < nch) {
                fetch(ch + 1, k, rk);
                fetch(ch + 1, v, rv);
            }
            __syncthreads();
            const int j = ch * S8_CH + sk;
            double u = 0.0, sj = 0.0;   // (k_j - kbar).y and q.k_j over this thread's 32 features
#pragma unroll 8
            for (int e = 0; e < 32; ++e) {
                const int a = 32 * sq + e;
                const double kv = bf2d(KC[sk * S8_KLD + a]);
                u = fma(kv - KB[a], YS[a], u);
                sj = fma(QS[a], kv, sj);
            }
            u += __shfl_xor(u, 1);
            u += __shfl_xor(u, 2);
            sj += __shfl_xor(sj, 1);
            sj += __shfl_xor(sj, 2);
            // w_j recomputed with pass 1's arithmetic (the same sum order, then exp(s - m))
            if (sq == 0) WU[sk] = j < nk ? exp(sj * inv_h - m) * u : 0.0;
            __syncthreads();
            for (int kk = par; kk < S8_CH; kk += 2) {
                const double wu = WU[kk];
                acc_o = fma(wu, bf2d(VC[kk * S8_KLD + f]), acc_o);
                swu += wu;
            }
        }
    }
    __syncthreads();
    PART[par * SD + f] = acc_o;
    __syncthreads();
    const double accf = PART[f] + PART[SD + f];
    __syncthreads();
    PART[par * SD + f] = swu;
    __syncthreads();
    if (tid < SD) {
        const double sw_all = PART[f] + PART[SD + f];
        out[base + static_cast<int64_t>(i) * SD + f] = static_cast<float>(VB[f] - (accf - VB[f] * sw_all));
    }
}

template <int W>
__device__ __forceinline__ void s8_chunk(double4v (&acc)[9], const uint16_t* __restrict__ kc,
                                         const double* __restrict__ sw, const double (&kbf)[8], int nst,
                                         int g, int c) {
    for (int st = 0; st < nst; ++st) {
        const int jl = 4 * st + g;
        const double swj = sw[jl];
        const uint16_t* kr = kc + jl * S8_KLD + c;
        double r[8];
#pragma unroll
        for (int F = 0; F < 8; ++F) r[F] = s8_uses(W, F) ? swj * (bf2d(kr[16 * F]) - kbf[F]) : 0.0;
#pragma unroll
        for (int b = 0; b < 9; ++b)
            acc[b] = __builtin_amdgcn_mfma_f64_16x16x4f64(r[s8_bi[W][b]], r[s8_bj[W][b]], acc[b], 0, 0, 0);
    }
}

}  // namespace

hipError_t launch_short128(const Problem& p, int rows) {
    if (rows <= 0) return hipSuccess;
    if (p.d != SD || p.dtype != 1 || rows > S8_MAXK) return hipErrorInvalidValue;
    const int BH = static_cast<int>(p.B * p.H);
    prof_begin(p.stream, "lla8_short_kernel");
    lla8_short_kernel<<<dim3(static_cast<unsigned>(BH) * static_cast<unsigned>(rows)), dim3(256), 0, p.stream>>>(
        static_cast<const uint16_t*>(p.q), static_cast<const uint16_t*>(p.k), static_cast<const uint16_t*>(p.v), p.out,
        static_cast<int>(p.n), rows, BH, 1.0 / p.h, p.lambda);
    prof_end(p.stream);
    return hipGetLastError();
}

}  // namespace lla
