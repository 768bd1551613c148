// Backward of the causal Parallax forward with a caller-supplied probe: the gradients of
// sum(o * dout) with respect to q, k, v and rho.
//
// ("Parallax" blog post, Appendix F "Parallax backward": a row-tile pass and a column-tile
// pass over cached row statistics.  The page's formulas are stripped; the closed form below
// is derived from the scoring form of the forward, o_i = sum_j a_ij v_j with
// a_ij = p_ij (1 - u_ij + ubar_i), u_ij = rho_i . k_j, ubar_i = sum_j p_ij u_ij = rho_i . kbar_i,
// p_ij = softmax_j(q_i . k_j / h) over j <= i.)
//
//   g_ij  = dout_i . v_j,            G_i = sum_j p_ij g_ij = dout_i . vbar_i,
//   dp_ij = g_ij (1 - u_ij + ubar_i) + u_ij G_i,
//   D_i   = sum_j p_ij dp_ij = dout_i . o_i + ubar_i G_i,
//   ds_ij = p_ij (dp_ij - D_i),       du_ij = p_ij (G_i - g_ij),
//   dq_i  = sum_j ds_ij k_j / h,      drho_i = sum_j du_ij k_j,
//   dk_j  = sum_i (ds_ij q_i / h + du_ij rho_i),   dv_j = sum_i a_ij dout_i.
//
// Matrix-core path (bf16, d = 64; needs the forward's per-row log-sum-exp as a shift):
//   lla_parallax_bwd_pack_kernel  per 64-position tile: a query image (q, rho, dout row-major
//                                 and feature-major, and a float4 of row statistics) and a
//                                 key image (k, v row-major, k feature-major), bf16.
//   lla_parallax_bwd_qr_kernel<true>  statistics sweep over each row's keys with the same
//                                 products as the passes below: Z = sum e, sum e u, sum e g,
//                                 sum e g u with e = 2^(x - lse_fwd); then lse = lse_fwd +
//                                 log2 Z, ubar, G and D = G (1 + 2 ubar) - sum p g u replace
//                                 the row statistics.  D and the normaliser must be those of
//                                 the p, u, g the passes use: dq_i = sum_j ds_ij k_j / h with
//                                 sum_j ds_ij = 0, and an inconsistent D (one taken from the
//                                 forward's rounded weights) leaves D-error times kbar in dq.
//   lla_parallax_bwd_kv_kernel    column pass: a block owns 128 keys (16 per wave) and
//                                 streams the query images of rows >= its first key through
//                                 LDS: S = Q K^T, U = R K^T, g = dout V^T (bf16 MFMA), then
//                                 a, ds/h, du per pair, and dv^T += dout^T a,
//                                 dk^T += Q^T ds/h + R^T du.
//   lla_parallax_bwd_qr_kernel<false>  row pass: a block owns 128 rows (16 per wave) and streams
//                                 the key images of keys <= its last row: S^T, U^T, g^T, then
//                                 dq += (ds/h) K and drho += du K.
// The weights a, ds, du enter the accumulating products as bf16 hi + lo pairs (two MFMAs,
// about 16 significant bits) against exact bf16 operands: no fp16 range limit anywhere.
//
// fp64 path (every dtype and d): lla_parallax_bwd_exact_rows_kernel (one block per row: the
// row's statistics in fp64 from scratch, then dq and drho) and
// lla_parallax_bwd_exact_cols_kernel (one block per key: dk and dv over the rows >= it).
#include "lla_device.h"
#include "lla_internal.h"

#include <math.h>

#include <mutex>
#include <type_traits>

namespace lla {
namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int BT = 64;                          // rows or keys per tile
constexpr int R_LD = FD + 8;                    // row-major bf16 row, halves (144 B)
constexpr int T_LD = BT + 4;                    // feature-major bf16 row, halves (136 B = 34 banks)
constexpr int RM_BYTES = BT * R_LD * 2;         // 9216
constexpr int TM_BYTES = FD * T_LD * 2;         // 8704
// Query image: q, rho, dout row-major | q, rho, dout feature-major | row statistics
// (lse, 1 + ubar, G, D) as one float4 per row.
constexpr int QI_Q = 0, QI_R = RM_BYTES, QI_D = 2 * RM_BYTES;
constexpr int QI_QT = 3 * RM_BYTES, QI_RT = QI_QT + TM_BYTES, QI_DT = QI_RT + TM_BYTES;
constexpr int QI_ST = QI_DT + TM_BYTES;
constexpr int QIMG = (QI_ST + BT * 16 + 1023) / 1024 * 1024;   // 55296
// Key image: k, v row-major | k feature-major.
constexpr int KI_K = 0, KI_V = RM_BYTES, KI_KT = 2 * RM_BYTES;
constexpr int KIMG = (KI_KT + TM_BYTES + 1023) / 1024 * 1024;  // 27648
constexpr int BW = 8;                           // waves per block in both passes
constexpr int BNT = BW * 64;
constexpr int BROWS = 16 * BW;                  // keys (column pass) or rows (row pass) per block
constexpr int KV_NBUF = 2;                      // query images in LDS in the column pass (1 measured slower)

// ---------------------------------------------------------------------------------------
// Pack: block per (head, tile), thread -> row r = tid / 4 of the tile, features 16 fc ..
// 16 fc + 15 (fc = tid % 4); the transposes go through LDS.  Rows past n are zero with
// lse = +inf, so every weight of such a row is 0.
__global__ __launch_bounds__(256) void lla_parallax_bwd_pack_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ rho, const uint16_t* __restrict__ dout, const float* __restrict__ lse_fwd,
    unsigned char* __restrict__ qimg, unsigned char* __restrict__ kimg, int n, int ntiles) {
    __shared__ uint16_t tr[4][BT][FD + 2];   // q, rho, dout, k of the tile
    const int tid = threadIdx.x;
    const int bh = static_cast<int>(blockIdx.x) / ntiles, t = static_cast<int>(blockIdx.x) % ntiles;
    const int r = tid >> 2, fc = tid & 3;
    const int i = t * BT + r;
    const bool in = i < n;
    const int64_t row = static_cast<int64_t>(bh) * n + i;
    unsigned char* qi = qimg + (static_cast<int64_t>(bh) * ntiles + t) * QIMG;
    unsigned char* ki = kimg + (static_cast<int64_t>(bh) * ntiles + t) * KIMG;
    const uint16_t* srcs[5] = {q, rho, dout, k, v};
    unsigned char* dsts[5] = {qi + QI_Q, qi + QI_R, qi + QI_D, ki + KI_K, ki + KI_V};
#pragma unroll
    for (int a = 0; a < 5; ++a) {
        uint4 x0 = {0u, 0u, 0u, 0u}, x1 = {0u, 0u, 0u, 0u};
        if (in) {
            const uint4* src = reinterpret_cast<const uint4*>(srcs[a] + row * FD + 16 * fc);
            x0 = src[0];
            x1 = src[1];
        }
        uint4* dst = reinterpret_cast<uint4*>(dsts[a] + r * (R_LD * 2) + 32 * fc);
        dst[0] = x0;
        dst[1] = x1;
        if (a < 4) {
            const uint32_t w[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                tr[a][r][16 * fc + 2 * e] = static_cast<uint16_t>(w[e] & 0xffffu);
                tr[a][r][16 * fc + 2 * e + 1] = static_cast<uint16_t>(w[e] >> 16);
            }
        }
    }
    // Row statistics: the forward's log-sum-exp as the shift of the statistics sweep.
    if (fc == 0)
        *reinterpret_cast<float4v*>(qi + QI_ST + r * 16) = float4v{in ? lse_fwd[row] : INFINITY, 0.0f, 0.0f, 0.0f};
    __syncthreads();
    // Feature-major copies: thread -> feature f, rows 16 rc .. 16 rc + 15.
    const int f = tid >> 2, rc = tid & 3;
    unsigned char* tdst[4] = {qi + QI_QT, qi + QI_RT, qi + QI_DT, ki + KI_KT};
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        uint32_t w[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            w[e] = static_cast<uint32_t>(tr[a][16 * rc + 2 * e][f]) |
                   (static_cast<uint32_t>(tr[a][16 * rc + 2 * e + 1][f]) << 16);
        uint4* dst = reinterpret_cast<uint4*>(tdst[a] + f * (T_LD * 2) + 32 * rc);
        dst[0] = uint4{w[0], w[1], w[2], w[3]};
        dst[1] = uint4{w[4], w[5], w[6], w[7]};
    }
}

// Whole-image copies global -> registers -> LDS, 16 bytes per thread per round; the
// threads past the image's last chunk copy that chunk again (same bytes, same place).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <int IMG>
struct ImageCopy {
    static constexpr int CH = IMG / 16, PT = (CH + BNT - 1) / BNT;
    u32x4 pre[PT];
    __device__ __forceinline__ void fetch(const unsigned char* src, int tid) {
#pragma unroll
        for (int e = 0; e < PT; ++e) pre[e] = reinterpret_cast<const u32x4*>(src)[min(tid + BNT * e, CH - 1)];
    }
    __device__ __forceinline__ void stash(unsigned char* dst, int tid) const {
#pragma unroll
        for (int e = 0; e < PT; ++e) reinterpret_cast<u32x4*>(dst)[min(tid + BNT * e, CH - 1)] = pre[e];
    }
};

// x as bf16 hi + lo (x - hi rounded again): about 16 significant bits together.
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {   // two values per conversion
        const f32x2 v = {x[2 * e], x[2 * e + 1]};
        h[e] = __builtin_convertvector(v, bf16x2);
        l[e] = __builtin_convertvector(v - __builtin_convertvector(h[e], f32x2), bf16x2);
    }
    hi = bf16x8{h[0][0], h[0][1], h[1][0], h[1][1], h[2][0], h[2][1], h[3][0], h[3][1]};
    lo = bf16x8{l[0][0], l[0][1], l[1][0], l[1][1], l[2][0], l[2][1], l[3][0], l[3][1]};
}

// 8 K-slots of a feature-major operand: rows (or keys) 4g .. 4g+3 and 16+4g .. 16+4g+3 of a
// 32-wide step, matching the accumulator layout of two stacked 16x16 score blocks.
__device__ __forceinline__ bf16x8 tpair(const unsigned char* p) {
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(p + 32);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ---------------------------------------------------------------------------------------
// Column pass.  Wave w owns keys kw0 .. kw0+15 (lane column c = key kw0 + c).  Per query
// tile, score blocks rb = 0..3 (rows 16 rb + 4g + r in register r).
template <int NBUF>   // query images held in LDS: 2 (one barrier per tile) or 1 (two blocks per CU)
__global__ __launch_bounds__(BNT, 1) void lla_parallax_bwd_kv_kernel(
    const unsigned char* __restrict__ qimg, const unsigned char* __restrict__ kimg, float* __restrict__ dk,
    float* __restrict__ dv, int n, int BH, int ntiles, float sl2, float inv_h) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c = lane & 15;
    const int nkb = (n + BROWS - 1) / BROWS;
    int bh, blk;
    head_major_block(static_cast<int>(blockIdx.x), BH, nkb, &bh, &blk);
    const int kblk = nkb - 1 - blk;                 // the first key blocks have the most rows
    const int j0 = kblk * BROWS;
    const int kw0 = j0 + 16 * wu;
    const int kc = kw0 + c;
    const int ktile = min(kc / BT, ntiles - 1);
    const unsigned char* kiw = kimg + (static_cast<int64_t>(bh) * ntiles + ktile) * KIMG;
    const int kr = kc - ktile * BT;                 // < BT whenever kc < n
    bf16x8 kb[2], vb[2];
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
        const int o = (kr & (BT - 1)) * (R_LD * 2) + 64 * ch + 16 * g;
        kb[ch] = *reinterpret_cast<const bf16x8*>(kiw + KI_K + o);
        vb[ch] = *reinterpret_cast<const bf16x8*>(kiw + KI_V + o);
    }
    float4v dvT[4], dkT[4];
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) {
        dvT[fb] = float4v{0.f, 0.f, 0.f, 0.f};
        dkT[fb] = float4v{0.f, 0.f, 0.f, 0.f};
    }
    const unsigned char* qih = qimg + static_cast<int64_t>(bh) * ntiles * QIMG;
    const int qt0 = j0 / BT;
    ImageCopy<QIMG> cp;
    cp.fetch(qih + static_cast<int64_t>(qt0) * QIMG, tid);
    cp.stash(lds, tid);
    __syncthreads();
    const float4v zero = {0.f, 0.f, 0.f, 0.f};
    for (int t = qt0; t < ntiles; ++t) {
        const int b = NBUF == 2 ? (t - qt0) & 1 : 0;
        if (t + 1 < ntiles) cp.fetch(qih + static_cast<int64_t>(t + 1) * QIMG, tid);
        const int i0 = t * BT;
        if (kw0 <= i0 + BT - 1 && kw0 < n) {   // wave-uniform: some row of the tile sees a key
            const unsigned char* img = lds + b * QIMG;
            float4v S[4], U[4], Gm[4];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int ro = (16 * rb + c) * (R_LD * 2) + 16 * g;
                const bf16x8 q0 = *reinterpret_cast<const bf16x8*>(img + QI_Q + ro);
                const bf16x8 q1 = *reinterpret_cast<const bf16x8*>(img + QI_Q + ro + 64);
                const bf16x8 r0 = *reinterpret_cast<const bf16x8*>(img + QI_R + ro);
                const bf16x8 r1 = *reinterpret_cast<const bf16x8*>(img + QI_R + ro + 64);
                const bf16x8 d0 = *reinterpret_cast<const bf16x8*>(img + QI_D + ro);
                const bf16x8 d1 = *reinterpret_cast<const bf16x8*>(img + QI_D + ro + 64);
                S[rb] = mfma_bf16(q1, kb[1], mfma_bf16(q0, kb[0], zero));
                U[rb] = mfma_bf16(r1, kb[1], mfma_bf16(r0, kb[0], zero));
                Gm[rb] = mfma_bf16(d1, vb[1], mfma_bf16(d0, vb[0], zero));
            }
            // pair weights of rows 32 ch .. 32 ch + 31; the causal mask only where the tile
            // reaches below the wave's last key
            auto weights = [&](auto masked, int ch, float (&av)[8], float (&sv)[8], float (&uv)[8]) {
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) {
                    const int rb = 2 * ch + hb;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int il = 16 * rb + 4 * g + r;
                        const float4v st = *reinterpret_cast<const float4v*>(img + QI_ST + il * 16);
                        float p = __builtin_amdgcn_exp2f(fmaf(S[rb][r], sl2, -st[0]));
                        if constexpr (decltype(masked)::value) p = i0 + il >= kc ? p : 0.0f;
                        const float u = U[rb][r], gg = Gm[rb][r];
                        const float t1 = st[1] - u;   // 1 - u + ubar
                        av[4 * hb + r] = p * t1;
                        sv[4 * hb + r] = p * (fmaf(gg, t1, fmaf(u, st[2], -st[3]))) * inv_h;
                        uv[4 * hb + r] = p * (st[2] - gg);
                    }
                }
            };
            const bool below = i0 >= kw0 + 15;   // every row of the tile sees every key of the wave
#pragma unroll
            for (int ch = 0; ch < 2; ++ch) {
                float av[8], sv[8], uv[8];
                if (below)
                    weights(std::false_type{}, ch, av, sv, uv);
                else
                    weights(std::true_type{}, ch, av, sv, uv);
                bf16x8 ah, al, sh, sl, uh, ul;
                split8(av, ah, al);
                split8(sv, sh, sl);
                split8(uv, uh, ul);
#pragma unroll
                for (int fb = 0; fb < 4; ++fb) {
                    const int to = (16 * fb + c) * (T_LD * 2) + (32 * ch + 4 * g) * 2;
                    const bf16x8 dt = tpair(img + QI_DT + to);
                    const bf16x8 qt = tpair(img + QI_QT + to);
                    const bf16x8 rt = tpair(img + QI_RT + to);
                    dvT[fb] = mfma_bf16(dt, al, mfma_bf16(dt, ah, dvT[fb]));
                    dkT[fb] = mfma_bf16(qt, sl, mfma_bf16(qt, sh, dkT[fb]));
                    dkT[fb] = mfma_bf16(rt, ul, mfma_bf16(rt, uh, dkT[fb]));
                }
            }
        }
        if constexpr (NBUF == 1) __syncthreads();   // every wave is done with the image
        if (t + 1 < ntiles) cp.stash(lds + (NBUF == 2 ? (b ^ 1) * QIMG : 0), tid);
        __syncthreads();
    }
    // lane (g, c) register r of block fb: feature 16 fb + 4g + r of key kc
    if (kc < n) {
        const int64_t o = (static_cast<int64_t>(bh) * n + kc) * FD + 4 * g;
#pragma unroll
        for (int fb = 0; fb < 4; ++fb) {
            *reinterpret_cast<float4v*>(dk + o + 16 * fb) = dkT[fb];
            *reinterpret_cast<float4v*>(dv + o + 16 * fb) = dvT[fb];
        }
    }
}

// ---------------------------------------------------------------------------------------
// Row pass.  Wave w owns rows iw0 .. iw0+15 (lane column c = row iw0 + c in the score
// blocks S^T[key 16 kb + 4g + r][row]).
template <bool kSweep>   // true: the statistics sweep (writes the row statistics, no gradients)
__global__ __launch_bounds__(BNT, 1) void lla_parallax_bwd_qr_kernel(
    unsigned char* __restrict__ qimg, const unsigned char* __restrict__ kimg, float* __restrict__ dq,
    float* __restrict__ drho, int n, int BH, int ntiles, float sl2, float inv_h) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c = lane & 15;
    const int nrb = (n + BROWS - 1) / BROWS;
    int bh, blk;
    head_major_block(static_cast<int>(blockIdx.x), BH, nrb, &bh, &blk);   // longest first
    const int i0b = blk * BROWS;
    const int iw0 = i0b + 16 * wu;
    const int ic = iw0 + c;
    const int qtile = min(ic / BT, ntiles - 1);
    unsigned char* qiw = qimg + (static_cast<int64_t>(bh) * ntiles + qtile) * QIMG;
    const int ir = (ic - qtile * BT) & (BT - 1);
    bf16x8 qb[2], rb_[2], db[2];
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
        const int o = ir * (R_LD * 2) + 64 * ch + 16 * g;
        qb[ch] = *reinterpret_cast<const bf16x8*>(qiw + QI_Q + o);
        rb_[ch] = *reinterpret_cast<const bf16x8*>(qiw + QI_R + o);
        db[ch] = *reinterpret_cast<const bf16x8*>(qiw + QI_D + o);
    }
    const float4v st = *reinterpret_cast<const float4v*>(qiw + QI_ST + ir * 16);   // lse, 1 + ubar, G, D (after the sweep)
    float4v dqa[4], dra[4];
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) {
        dqa[fb] = float4v{0.f, 0.f, 0.f, 0.f};
        dra[fb] = float4v{0.f, 0.f, 0.f, 0.f};
    }
    float z = 0.0f, zu = 0.0f, zg = 0.0f, zgu = 0.0f;   // statistics sweep sums of this lane
    const unsigned char* kih = kimg + static_cast<int64_t>(bh) * ntiles * KIMG;
    const int tl = min(ntiles - 1, (min(i0b + BROWS, n) - 1) / BT);
    ImageCopy<KIMG> cp;
    cp.fetch(kih, tid);
    cp.stash(lds, tid);
    __syncthreads();
    const float4v zero = {0.f, 0.f, 0.f, 0.f};
    for (int t = 0; t <= tl; ++t) {
        const int b = t & 1;
        if (t + 1 <= tl) cp.fetch(kih + static_cast<int64_t>(t + 1) * KIMG, tid);
        const int j0 = t * BT;
        if (iw0 + 15 >= j0 && iw0 < n) {   // wave-uniform: some row of the wave sees a key
            const unsigned char* img = lds + b * KIMG;
            float4v S[4], U[4], Gm[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int ro = (16 * kb + c) * (R_LD * 2) + 16 * g;
                const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(img + KI_K + ro);
                const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(img + KI_K + ro + 64);
                const bf16x8 v0 = *reinterpret_cast<const bf16x8*>(img + KI_V + ro);
                const bf16x8 v1 = *reinterpret_cast<const bf16x8*>(img + KI_V + ro + 64);
                S[kb] = mfma_bf16(k1, qb[1], mfma_bf16(k0, qb[0], zero));
                U[kb] = mfma_bf16(k1, rb_[1], mfma_bf16(k0, rb_[0], zero));
                Gm[kb] = mfma_bf16(v1, db[1], mfma_bf16(v0, db[0], zero));
            }
            if constexpr (kSweep) {
                auto sums = [&](auto masked) {
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int j = j0 + 16 * kb + 4 * g + r;
                            float e = __builtin_amdgcn_exp2f(fmaf(S[kb][r], sl2, -st[0]));
                            if constexpr (decltype(masked)::value) e = j <= ic ? e : 0.0f;
                            const float eg = e * Gm[kb][r];
                            z += e;
                            zu = fmaf(e, U[kb][r], zu);
                            zg += eg;
                            zgu = fmaf(eg, U[kb][r], zgu);
                        }
                };
                if (j0 + BT - 1 <= iw0)   // every row of the wave sees every key of the tile
                    sums(std::false_type{});
                else
                    sums(std::true_type{});
            } else
            {
            // pair weights of keys 32 ch .. 32 ch + 31 (ds without its 1/h, applied to dq at the
            // end); the causal mask only where the tile reaches past the wave's first row
            auto weights = [&](auto masked, int ch, float (&sv)[8], float (&uv)[8]) {
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) {
                    const int kb = 2 * ch + hb;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = j0 + 16 * kb + 4 * g + r;
                        float p = __builtin_amdgcn_exp2f(fmaf(S[kb][r], sl2, -st[0]));
                        if constexpr (decltype(masked)::value) p = j <= ic ? p : 0.0f;
                        const float u = U[kb][r], gg = Gm[kb][r];
                        const float t1 = st[1] - u;   // 1 - u + ubar
                        sv[4 * hb + r] = p * fmaf(gg, t1, fmaf(u, st[2], -st[3]));
                        uv[4 * hb + r] = p * (st[2] - gg);
                    }
                }
            };
            const bool below = j0 + BT - 1 <= iw0;   // every row of the wave sees every key of the tile
#pragma unroll
            for (int ch = 0; ch < 2; ++ch) {
                float sv[8], uv[8];
                if (below)
                    weights(std::false_type{}, ch, sv, uv);
                else
                    weights(std::true_type{}, ch, sv, uv);
                bf16x8 sh, sl, uh, ul;
                split8(sv, sh, sl);
                split8(uv, uh, ul);
#pragma unroll
                for (int fb = 0; fb < 4; ++fb) {
                    const bf16x8 kt = tpair(img + KI_KT + (16 * fb + c) * (T_LD * 2) + (32 * ch + 4 * g) * 2);
                    dqa[fb] = mfma_bf16(sl, kt, mfma_bf16(sh, kt, dqa[fb]));
                    dra[fb] = mfma_bf16(ul, kt, mfma_bf16(uh, kt, dra[fb]));
                }
            }
            }
        }
        if (t + 1 <= tl) cp.stash(lds + (b ^ 1) * KIMG, tid);
        __syncthreads();
    }
    if constexpr (kSweep) {
        // row ic's sums are spread over the lane groups g: combine, then lane g = 0 writes
        // lse, 1 + ubar, G, D of the row into its query image
        z += __shfl_xor(z, 16);
        z += __shfl_xor(z, 32);
        zu += __shfl_xor(zu, 16);
        zu += __shfl_xor(zu, 32);
        zg += __shfl_xor(zg, 16);
        zg += __shfl_xor(zg, 32);
        zgu += __shfl_xor(zgu, 16);
        zgu += __shfl_xor(zgu, 32);
        if (g == 0 && ic < n) {
            const float iz = 1.0f / z, ub = zu * iz, G = zg * iz;
            *reinterpret_cast<float4v*>(qiw + QI_ST + ir * 16) =
                float4v{st[0] + __log2f(z), 1.0f + ub, G, fmaf(G, 1.0f + 2.0f * ub, -zgu * iz)};
        }
        return;
    }
    // lane (g, c) register r of block fb: row iw0 + 4g + r, feature 16 fb + c
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = iw0 + 4 * g + r;
        if (i < n) {
            const int64_t o = (static_cast<int64_t>(bh) * n + i) * FD + c;
#pragma unroll
            for (int fb = 0; fb < 4; ++fb) {
                dq[o + 16 * fb] = dqa[fb][r] * inv_h;
                drho[o + 16 * fb] = dra[fb][r];
            }
        }
    }
}

// ---------------------------------------------------------------------------------------
// fp64 path.

constexpr int EB_NT = 256;
constexpr int EB_CHK = 256;

__device__ __forceinline__ double eb_reduce(double x, bool is_max, double* red) {
    const int tid = threadIdx.x;
    red[tid] = x;
    __syncthreads();
    for (int s = EB_NT / 2; s > 0; s >>= 1) {
        if (tid < s) red[tid] = is_max ? fmax(red[tid], red[tid + s]) : red[tid] + red[tid + s];
        __syncthreads();
    }
    const double r = red[0];
    __syncthreads();
    return r;
}

// Sum over the key lanes kl of red[kl * D + f] for f = tid < D (after a barrier).
template <int D>
__device__ __forceinline__ double eb_feature_sum(double x, double* red) {
    constexpr int KL = EB_NT / D;
    const int tid = threadIdx.x;
    red[tid] = x;
    __syncthreads();
    double s = 0.0;
    if (tid < D)
        for (int l = 0; l < KL; ++l) s += red[l * D + tid];
    __syncthreads();
    return s;
}

// Block per row i: the row's statistics in fp64 (max, omega, kbar, vbar, then
// ubar = rho . kbar, G = dout . vbar, D = sum_j p dp), then dq and drho; writes
// (m + log omega, ubar, G, D) to rst for the column kernel.
template <typename TIn, int D>
__global__ __launch_bounds__(EB_NT) void lla_parallax_bwd_exact_rows_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v, const TIn* __restrict__ rho,
    const TIn* __restrict__ dout, float* __restrict__ dq, float* __restrict__ drho, double* __restrict__ rst, int n,
    int BH, double inv_h) {
    constexpr int KL = EB_NT / D;
    __shared__ double qs[D], rs[D], os[D], kbar[D], vbar[D];
    __shared__ double c1[EB_CHK], c2[EB_CHK];
    __shared__ double red[EB_NT];
    const int tid = threadIdx.x;
    const int i = n - 1 - static_cast<int>(blockIdx.x / BH);   // longest rows first
    const int bh = static_cast<int>(blockIdx.x % BH);
    const int64_t base = static_cast<int64_t>(bh) * n * D;
    const int cnt = i + 1;
    for (int e = tid; e < D; e += EB_NT) {
        qs[e] = load_f64(q + base, static_cast<int64_t>(i) * D + e);
        rs[e] = load_f64(rho + base, static_cast<int64_t>(i) * D + e);
        os[e] = load_f64(dout + base, static_cast<int64_t>(i) * D + e);
    }
    __syncthreads();
    auto dot = [&](const double* a, const TIn* rowp, int j) {
        double s = 0.0;
#pragma unroll 8
        for (int e = 0; e < D; ++e) s += a[e] * load_f64(rowp + base, static_cast<int64_t>(j) * D + e);
        return s;
    };
    double mloc = -INFINITY;
    for (int j = tid; j < cnt; j += EB_NT) mloc = fmax(mloc, dot(qs, k, j) * inv_h);
    const double m = eb_reduce(mloc, true, red);
    const int fa = tid % D, kl = tid / D;
    double aw = 0.0, ak = 0.0, av = 0.0;
    for (int c0 = 0; c0 < cnt; c0 += EB_CHK) {
        const int nk = min(EB_CHK, cnt - c0);
        if (tid < nk) c1[tid] = exp(dot(qs, k, c0 + tid) * inv_h - m);
        __syncthreads();
        for (int jj = kl; jj < nk; jj += KL) {
            const int64_t off = static_cast<int64_t>(c0 + jj) * D + fa;
            ak += c1[jj] * load_f64(k + base, off);
            av += c1[jj] * load_f64(v + base, off);
        }
        if (tid < nk) aw += c1[tid];
        __syncthreads();
    }
    const double omega = eb_reduce(aw, false, red);
    const double skb = eb_feature_sum<D>(ak, red);
    const double svb = eb_feature_sum<D>(av, red);
    if (tid < D) {
        kbar[tid] = skb / omega;
        vbar[tid] = svb / omega;
    }
    __syncthreads();
    double ub = 0.0, G = 0.0;
    for (int e = 0; e < D; ++e) {
        ub += rs[e] * kbar[e];
        G += os[e] * vbar[e];
    }
    // D = sum_j p dp
    double ad = 0.0;
    for (int j = tid; j < cnt; j += EB_NT) {
        const double p = exp(dot(qs, k, j) * inv_h - m) / omega;
        const double u = dot(rs, k, j), gg = dot(os, v, j);
        ad += p * (gg * (1.0 - u + ub) + u * G);
    }
    const double Dd = eb_reduce(ad, false, red);
    // dq = sum_j ds k_j / h, drho = sum_j du k_j
    double aq = 0.0, ar = 0.0;
    for (int c0 = 0; c0 < cnt; c0 += EB_CHK) {
        const int nk = min(EB_CHK, cnt - c0);
        if (tid < nk) {
            const int j = c0 + tid;
            const double p = exp(dot(qs, k, j) * inv_h - m) / omega;
            const double u = dot(rs, k, j), gg = dot(os, v, j);
            c1[tid] = p * (gg * (1.0 - u + ub) + u * G - Dd) * inv_h;
            c2[tid] = p * (G - gg);
        }
        __syncthreads();
        for (int jj = kl; jj < nk; jj += KL) {
            const double kv = load_f64(k + base, static_cast<int64_t>(c0 + jj) * D + fa);
            aq += c1[jj] * kv;
            ar += c2[jj] * kv;
        }
        __syncthreads();
    }
    const double sq = eb_feature_sum<D>(aq, red);
    const double sr = eb_feature_sum<D>(ar, red);
    if (tid < D) {
        dq[base + static_cast<int64_t>(i) * D + tid] = static_cast<float>(sq);
        drho[base + static_cast<int64_t>(i) * D + tid] = static_cast<float>(sr);
    }
    if (tid == 0) {
        double* o = rst + (static_cast<int64_t>(bh) * n + i) * 4;
        o[0] = m + log(omega);
        o[1] = ub;
        o[2] = G;
        o[3] = Dd;
    }
}

// Block per key j: dk_j = sum_{i >= j} (ds_ij q_i / h + du_ij rho_i), dv_j = sum_{i >= j} a_ij dout_i,
// from the rows' fp64 statistics.
template <typename TIn, int D>
__global__ __launch_bounds__(EB_NT) void lla_parallax_bwd_exact_cols_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v, const TIn* __restrict__ rho,
    const TIn* __restrict__ dout, const double* __restrict__ rst, float* __restrict__ dk, float* __restrict__ dv,
    int n, int BH, double inv_h) {
    constexpr int KL = EB_NT / D;
    __shared__ double ks[D], vs[D];
    __shared__ double ca[EB_CHK], cs[EB_CHK], cu[EB_CHK];
    __shared__ double red[EB_NT];
    const int tid = threadIdx.x;
    const int j = static_cast<int>(blockIdx.x / BH);   // the first keys have the most rows
    const int bh = static_cast<int>(blockIdx.x % BH);
    const int64_t base = static_cast<int64_t>(bh) * n * D;
    for (int e = tid; e < D; e += EB_NT) {
        ks[e] = load_f64(k + base, static_cast<int64_t>(j) * D + e);
        vs[e] = load_f64(v + base, static_cast<int64_t>(j) * D + e);
    }
    __syncthreads();
    auto dot = [&](const double* a, const TIn* rowp, int i) {
        double s = 0.0;
#pragma unroll 8
        for (int e = 0; e < D; ++e) s += a[e] * load_f64(rowp + base, static_cast<int64_t>(i) * D + e);
        return s;
    };
    const int fa = tid % D, kl = tid / D;
    double akq = 0.0, akr = 0.0, avd = 0.0;
    for (int c0 = j; c0 < n; c0 += EB_CHK) {
        const int nr = min(EB_CHK, n - c0);
        if (tid < nr) {
            const int i = c0 + tid;
            const double* st = rst + (static_cast<int64_t>(bh) * n + i) * 4;
            const double p = exp(dot(ks, q, i) * inv_h - st[0]);
            const double u = dot(ks, rho, i), gg = dot(vs, dout, i);
            const double t1 = 1.0 - u + st[1];
            ca[tid] = p * t1;
            cs[tid] = p * (gg * t1 + u * st[2] - st[3]) * inv_h;
            cu[tid] = p * (st[2] - gg);
        }
        __syncthreads();
        for (int ii = kl; ii < nr; ii += KL) {
            const int64_t off = static_cast<int64_t>(c0 + ii) * D + fa;
            akq += cs[ii] * load_f64(q + base, off);
            akr += cu[ii] * load_f64(rho + base, off);
            avd += ca[ii] * load_f64(dout + base, off);
        }
        __syncthreads();
    }
    const double sk = eb_feature_sum<D>(akq + akr, red);
    const double sv = eb_feature_sum<D>(avd, red);
    if (tid < D) {
        dk[base + static_cast<int64_t>(j) * D + tid] = static_cast<float>(sk);
        dv[base + static_cast<int64_t>(j) * D + tid] = static_cast<float>(sv);
    }
}

template <typename TIn, int D>
hipError_t launch_bwd_exact_t(const BwdProblem& b, void* workspace) {
    const Problem& p = b.p;
    const int BH = static_cast<int>(p.B * p.H);
    const int n = static_cast<int>(p.n);
    const unsigned blocks = static_cast<unsigned>(p.B * p.H * p.n);
    double* rst = static_cast<double*>(workspace);
    const auto* dout = static_cast<const TIn*>(b.dout);
    prof_begin(p.stream, "lla_parallax_bwd_exact_rows_kernel");
    lla_parallax_bwd_exact_rows_kernel<TIn, D><<<dim3(blocks), dim3(EB_NT), 0, p.stream>>>(
        static_cast<const TIn*>(p.q), static_cast<const TIn*>(p.k), static_cast<const TIn*>(p.v),
        static_cast<const TIn*>(p.rho), dout, b.dq, b.drho, rst, n, BH, 1.0 / p.h);
    prof_end(p.stream);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    prof_begin(p.stream, "lla_parallax_bwd_exact_cols_kernel");
    lla_parallax_bwd_exact_cols_kernel<TIn, D><<<dim3(blocks), dim3(EB_NT), 0, p.stream>>>(
        static_cast<const TIn*>(p.q), static_cast<const TIn*>(p.k), static_cast<const TIn*>(p.v),
        static_cast<const TIn*>(p.rho), dout, rst, b.dk, b.dv, n, BH, 1.0 / p.h);
    prof_end(p.stream);
    return hipGetLastError();
}

template <typename TIn>
hipError_t launch_bwd_exact_d(const BwdProblem& b, void* workspace) {
    switch (b.p.d) {
        case 16: return launch_bwd_exact_t<TIn, 16>(b, workspace);
        case 32: return launch_bwd_exact_t<TIn, 32>(b, workspace);
        case 64: return launch_bwd_exact_t<TIn, 64>(b, workspace);
        case 128: return launch_bwd_exact_t<TIn, 128>(b, workspace);
        default: return hipErrorInvalidValue;
    }
}

int64_t bwd_tiles(int64_t n) { return (n + BT - 1) / BT; }

}  // namespace

bool parallax_bwd_fast_supports(int dtype, int64_t d, int64_t n) {
    return dtype == 1 && d == FD && n <= kFastMaxN;
}

size_t parallax_bwd_workspace_bytes(int64_t B, int64_t H, int64_t n, int64_t d, bool fast) {
    (void)d;
    if (!fast) return static_cast<size_t>(B * H * n * 4 * 8);
    return static_cast<size_t>(B * H * bwd_tiles(n) * (QIMG + KIMG));
}

hipError_t launch_parallax_bwd_fast(const BwdProblem& b, void* workspace) {
    const Problem& p = b.p;
    const int n = static_cast<int>(p.n);
    const int BH = static_cast<int>(p.B * p.H);
    const int ntiles = static_cast<int>(bwd_tiles(p.n));
    unsigned char* qimg = static_cast<unsigned char*>(workspace);
    unsigned char* kimg = qimg + static_cast<int64_t>(BH) * ntiles * QIMG;
    {   // dynamic LDS above the default limit, raised once per device (the current one)
        static std::mutex attr_mu;
        static bool attr_done[64] = {};
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
        std::lock_guard<std::mutex> lock(attr_mu);
        if (!attr_done[dev]) {
            e = hipFuncSetAttribute(reinterpret_cast<const void*>(&lla_parallax_bwd_kv_kernel<KV_NBUF>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, KV_NBUF * QIMG);
            if (e == hipSuccess)
                e = hipFuncSetAttribute(reinterpret_cast<const void*>(&lla_parallax_bwd_qr_kernel<true>),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, 2 * KIMG);
            if (e == hipSuccess)
                e = hipFuncSetAttribute(reinterpret_cast<const void*>(&lla_parallax_bwd_qr_kernel<false>),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, 2 * KIMG);
            if (e != hipSuccess) return e;
            attr_done[dev] = true;
        }
    }
    prof_begin(p.stream, "lla_parallax_bwd_pack_kernel");
    lla_parallax_bwd_pack_kernel<<<dim3(static_cast<unsigned>(BH) * ntiles), dim3(256), 0, p.stream>>>(
        static_cast<const uint16_t*>(p.q), static_cast<const uint16_t*>(p.k), static_cast<const uint16_t*>(p.v),
        static_cast<const uint16_t*>(p.rho), static_cast<const uint16_t*>(b.dout), p.stats, qimg, kimg, n, ntiles);
    prof_end(p.stream);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const unsigned nblk = static_cast<unsigned>(BH) * static_cast<unsigned>((n + BROWS - 1) / BROWS);
    const float sl2 = static_cast<float>(LOG2E / p.h), inv_h = static_cast<float>(1.0 / p.h);
    prof_begin(p.stream, "lla_parallax_bwd_stats_kernel");
    lla_parallax_bwd_qr_kernel<true><<<dim3(nblk), dim3(BNT), 2 * KIMG, p.stream>>>(qimg, kimg, nullptr, nullptr, n,
                                                                                  BH, ntiles, sl2, inv_h);
    prof_end(p.stream);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    prof_begin(p.stream, "lla_parallax_bwd_kv_kernel");
    lla_parallax_bwd_kv_kernel<KV_NBUF><<<dim3(nblk), dim3(BNT), KV_NBUF * QIMG, p.stream>>>(qimg, kimg, b.dk, b.dv, n,
                                                                                          BH, ntiles, sl2, inv_h);
    prof_end(p.stream);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    prof_begin(p.stream, "lla_parallax_bwd_qr_kernel");
    lla_parallax_bwd_qr_kernel<false><<<dim3(nblk), dim3(BNT), 2 * KIMG, p.stream>>>(qimg, kimg, b.dq, b.drho, n, BH,
                                                                                   ntiles, sl2, inv_h);
    prof_end(p.stream);
    return hipGetLastError();
}

hipError_t launch_parallax_bwd_exact(const BwdProblem& b, void* workspace) {
    return b.p.dtype == 0 ? launch_bwd_exact_d<float>(b, workspace) : launch_bwd_exact_d<uint16_t>(b, workspace);
}

}  // namespace lla
