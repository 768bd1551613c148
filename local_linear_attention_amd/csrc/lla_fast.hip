// Matrix-core path of the causal LLA forward for bf16 inputs, head dimension 64.
//
// Work split (rows are query positions i of one head):
//   * rows i < 3d run in fp64 (the short-row blocks of lla_rows_kernel): their prefixes hold
//     at most 3d keys, so C_kk is rank-deficient or poorly conditioned and the ridge
//     lambda e^{-m} alone conditions the solve -- the normal-equation form then needs more
//     than fp16/fp32 precision (rows just past 2d still reach about 2e-3 in fp16);
//   * rows i >= 3d run here:
//       lla_anchor_kernel   per-head sums of the keys and values of positions [0, 2d) (the
//                           centring anchor a: every row of this path has them in its prefix);
//       lla_pack_kernel     K, V once into fp16 tiles centred at a (the LDS image the
//                           key-moment pass copies), K key-major for the score passes, and the
//                           check image (projected keys, |v - a_v|^2);
//       lla_rowmax_kernel   score pass with a running max: m_i;
//       lla_rows_kernel     the short rows, and per query, with sw_ij = sqrt(e^{s_ij - m_i})
//                           rounded to fp16 and R[j] = sw (k_j - a) (fp16), the key moment
//                           R^T R on MFMA (fp32 accumulation), the block sums
//                           S = sum_j sw^2 (k_j - a) and omega' = sum_j sw^2, the rank-one
//                           downdate to the centred C_kk and the ridge-rescaled SPD solve
//                           (C_kk + lambda e^{-m} I) y = kbar - q, kbar = a + S / omega';
//       lla_probe_kernel    b = vbar - C_vk y without forming C_vk (a second attention-like
//                           sweep over the keys and values), and the per-row check that hands
//                           rows to the fp64 kernel;
//       lla_exact_list_kernel  the rows handed back, in fp64.
// The estimator, its moments and the centred form follow the "Parallax" blog post, section 2
// "Canonical Formulation" and Appendix E; the max shift is the safe softmax of the arXiv
// page's scoring-form paragraph, with the ridge scaled by the same e^{-m}.  The normalisation
// by omega cancels in b, so unnormalised shifted weights serve throughout.
//
// MFMA: v_mfma_f32_16x16x32_{bf16,f16}.  Lane l supplies row/column (l % 16) of A/B and 8
// consecutive K-slots (l / 16); D[4 (l/16) + r][l % 16] lands in accumulator register r.
#include "lla_device.h"
#include "lla_internal.h"

#include <math.h>

#include <mutex>
#include <type_traits>

namespace lla {
namespace {

constexpr int B_WAVES = 4;          // waves per block of the row-max and key-moment passes

// ---------------------------------------------------------------------------------------
// Key tiles stream in 64-key tiles through a ring of three LDS buffers: tile t is consumed by
// the MFMAs while tile t+1 is landing and tile t+2 is being copied from the workspace straight
// into LDS (buffer loads with an LDS destination, no registers) -- one barrier per tile.
//
// Anchor: the pack kernel stores each head's keys and values centred at a = (mean k,
// mean v) of its positions [0, 2d) rounded to fp16 -- positions in the prefix of every row
// this path serves, so no row depends on a later position even through rounding -- and
// every wave only scales: R = sw (k - a).  Moments about a differ from the centred ones by a
// rank-one term,
//   C = sum_j w_j (k_j - a)(k_j - a)^T - S S^T / omega',   S = sum_j w_j (k_j - a),
// which the block gets from one extra MFMA per wave and 32 keys (weights w_j = sw_j^2 rounded
// to fp16, omega' their sum).  The cancellation in the downdate grows with |kbar_i - a|^2
// over the weighted spread of the keys, small while the query's weights are spread over many
// keys (as on RMS-normalised heads at h = sqrt(d)); the probe pass's check catches the rows
// where it is not.
constexpr int MT = 64;                   // keys per tile
constexpr int M_LD = MT + 8;             // feature-major fp16 row (elements), 144 B
// One tile as the pack kernel lays it out in the workspace (the key-moment pass copies its key
// half, the probe pass its value half, byte for byte, into LDS): [K or V][feature][key], rows
// of M_LD halves (the last 8 are
// padding that keeps the 16-byte operand reads conflict-free), 18 KiB per tile.
constexpr int PACK_TILE_BYTES = 2 * FD * M_LD * 2;
constexpr int M_NBUF = 3;                // tile ring: compute t, t+1 landing, t+2 in flight
constexpr int ANCHOR_SLICES = 16;        // key slices of the per-head anchor sums
// Keys of one tile key-major (bf16 as given, rows of KM_LD halves: 64 features + 8 of
// padding), the score operand of the row-max kernel, 9 KiB per tile.
constexpr int KM_LD = FD + 8;
constexpr int KM_TILE_BYTES = MT * KM_LD * 2;
// Workspace stride of a tile's key-major images: the bf16 keys, then the centred keys
// fp16(k - a) in the same layout.
constexpr int KM_STRIDE = 2 * KM_TILE_BYTES;
constexpr int KM_LOADS = KM_TILE_BYTES / 1024;
constexpr int KM_WLOADS = (KM_LOADS + B_WAVES - 1) / B_WAVES;
constexpr int R_SETS = 2, R_QW = 16 * R_SETS, R_QB = B_WAVES * R_QW;  // row-max: 2 sets of 16 queries per wave
static_assert(KM_TILE_BYTES % 1024 == 0, "key image must be whole wave copies");
static_assert(PACK_TILE_BYTES % 1024 == 0, "tile image must be whole wave copies");
// Check image of a tile: the centred keys projected on NCHK fixed +-1 directions (Walsh
// functions of odd index 2t + 1, fp16, feature-major [direction][key] rows of M_LD halves),
// then |v_j - a_v|^2 per key (fp32), padded to whole KiB.
constexpr int KU_NRM = NCHK * M_LD * 2;
static_assert(KU_NRM + MT * 4 <= KU_TILE_BYTES, "check image layout");

// Per-head anchor, pass 1: block (head, slice) sums its slice of the keys and values of
// positions [0, min(n, 2d)) per feature (fp32).  Thread -> 8 features (16 bytes) of K (groups 0-7) or V (groups 8-15) and
// every 16th key of the slice; the 16 key phases are then added up through LDS.
__global__ __launch_bounds__(256) void lla_anchor_kernel(const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v,
                                                         float* __restrict__ partial, unsigned* __restrict__ guard,
                                                         int n) {
    __shared__ float sums[16][2 * FD + 4];
    const int bh = static_cast<int>(blockIdx.x) / ANCHOR_SLICES;
    const int sl = static_cast<int>(blockIdx.x) % ANCHOR_SLICES;
    const int tid = threadIdx.x, fgrp = tid & 15, ph = tid >> 4;
    if (sl == 0 && tid < 2) guard[1 + 2 * bh + tid] = 0u;   // the head's range maxima
    if (blockIdx.x == 0 && tid == 2) guard[0] = 0u;         // no rows handed back yet
    const int na = min(n, 2 * FD);
    const int len = (na + ANCHOR_SLICES - 1) / ANCHOR_SLICES;
    const int j_lo = sl * len, j_hi = min(na, j_lo + len);
    const uint16_t* src = (fgrp < 8 ? k : v) + static_cast<int64_t>(bh) * n * FD + 8 * (fgrp & 7);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = j_lo + ph; j < j_hi; j += 16) {
        const uint4 x = *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(j) * FD);
        const uint32_t wds[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[e] += __uint_as_float((e & 1) ? (wds[e >> 1] & 0xffff0000u) : (wds[e >> 1] << 16));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) sums[ph][8 * fgrp + e] = acc[e];
    __syncthreads();
    if (tid < 2 * FD) {
        float tot = 0.0f;
#pragma unroll
        for (int q2 = 0; q2 < 16; ++q2) tot += sums[q2][tid];
        partial[(static_cast<int64_t>(bh) * ANCHOR_SLICES + sl) * 2 * FD + tid] = tot;
    }
}

// Pack K and V once into the LDS image of each tile (zero past n), centred at the head's
// anchor a = fp16(mean of k, of v over positions [0, 2d)): stored value fp16(x - a), one
// rounding.
// Thread -> keys 2p, 2p+1 and features 8fg .. 8fg+7; every store writes a pair of keys.
// The same block also writes the tile's keys key-major, as given (bf16) and centred
// (fp16(k - a), the same values as the feature-major image), and block 0 of each head the
// head's anchor (fp16 values as floats).
__global__ __launch_bounds__(256) void lla_pack_kernel(const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ v,
                                                       const float* __restrict__ partial,
                                                       float* __restrict__ anchors,
                                                       unsigned char* __restrict__ packed,
                                                       unsigned char* __restrict__ kimg,
                                                       unsigned char* __restrict__ kuimg,
                                                       unsigned* __restrict__ guard, int n,
                                                       int ntiles) {
    __shared__ float anc[2 * FD];
    __shared__ float ys[MT][8][5];      // per key and feature group: odd-index 8-point transforms
    __shared__ float vpart[8][MT];      // |v - a_v|^2 over each thread's 8 features
    __shared__ float wmax[4][2];        // per wave: largest |k - a|, |v - a_v|
    const int bh = static_cast<int>(blockIdx.x) / ntiles, t = static_cast<int>(blockIdx.x) % ntiles;
    const int tid = threadIdx.x, pr = tid & 31, fg = tid >> 5;
    if (tid < 2 * FD) {
        float sum = 0.0f;
        for (int sl = 0; sl < ANCHOR_SLICES; ++sl)
            sum += partial[(static_cast<int64_t>(bh) * ANCHOR_SLICES + sl) * 2 * FD + tid];
        anc[tid] = static_cast<float>(static_cast<_Float16>(sum / static_cast<float>(min(n, 2 * FD))));
        if (t == 0) anchors[static_cast<int64_t>(bh) * 2 * FD + tid] = anc[tid];
    }
    const int64_t base = static_cast<int64_t>(bh) * n * FD;
    const int ja = t * MT + 2 * pr, jb = ja + 1;
    uint4 k0 = make_uint4(0, 0, 0, 0), k1 = k0, v0 = k0, v1 = k0;
    if (ja < n) {
        k0 = *reinterpret_cast<const uint4*>(k + base + static_cast<int64_t>(ja) * FD + 8 * fg);
        v0 = *reinterpret_cast<const uint4*>(v + base + static_cast<int64_t>(ja) * FD + 8 * fg);
    }
    if (jb < n) {
        k1 = *reinterpret_cast<const uint4*>(k + base + static_cast<int64_t>(jb) * FD + 8 * fg);
        v1 = *reinterpret_cast<const uint4*>(v + base + static_cast<int64_t>(jb) * FD + 8 * fg);
    }
    {   // key-major image: key 2p (and 2p+1), features 8fg .. 8fg+7; row padding zero
        unsigned char* kt = kimg + (static_cast<int64_t>(bh) * ntiles + t) * KM_STRIDE;
        *reinterpret_cast<uint4*>(kt + (2 * pr) * (KM_LD * 2) + 16 * fg) = k0;
        *reinterpret_cast<uint4*>(kt + (2 * pr + 1) * (KM_LD * 2) + 16 * fg) = k1;
        if (fg == 0) {
            *reinterpret_cast<uint4*>(kt + (2 * pr) * (KM_LD * 2) + 2 * FD) = make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4*>(kt + (2 * pr + 1) * (KM_LD * 2) + 2 * FD) = make_uint4(0, 0, 0, 0);
        }
    }
    __syncthreads();
    {   // centred keys fp16(k - a), key-major, after the bf16 image; row padding zero
        unsigned char* kt = kimg + (static_cast<int64_t>(bh) * ntiles + t) * KM_STRIDE + KM_TILE_BYTES;
        const uint32_t wa[4] = {k0.x, k0.y, k0.z, k0.w}, wb[4] = {k1.x, k1.y, k1.z, k1.w};
        half8 ca, cb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float ak = anc[8 * fg + e];
            const uint32_t xa = wa[e >> 1], xb = wb[e >> 1];
            ca[e] = static_cast<_Float16>(ja >= n ? 0.0f : __uint_as_float((e & 1) ? (xa & 0xffff0000u) : (xa << 16)) - ak);
            cb[e] = static_cast<_Float16>(jb >= n ? 0.0f : __uint_as_float((e & 1) ? (xb & 0xffff0000u) : (xb << 16)) - ak);
        }
        *reinterpret_cast<half8*>(kt + (2 * pr) * (KM_LD * 2) + 16 * fg) = ca;
        *reinterpret_cast<half8*>(kt + (2 * pr + 1) * (KM_LD * 2) + 16 * fg) = cb;
        if (fg == 0) {
            *reinterpret_cast<uint4*>(kt + (2 * pr) * (KM_LD * 2) + 2 * FD) = make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4*>(kt + (2 * pr + 1) * (KM_LD * 2) + 2 * FD) = make_uint4(0, 0, 0, 0);
        }
    }
    uint32_t* dst = reinterpret_cast<uint32_t*>(packed + (static_cast<int64_t>(bh) * ntiles + t) * PACK_TILE_BYTES);
    const uint32_t ka[4] = {k0.x, k0.y, k0.z, k0.w}, kb[4] = {k1.x, k1.y, k1.z, k1.w};
    const uint32_t va[4] = {v0.x, v0.y, v0.z, v0.w}, vb[4] = {v1.x, v1.y, v1.z, v1.w};
    const bool za = ja >= n, zb = jb >= n;
    float vsa = 0.0f, vsb = 0.0f;   // |v - a_v|^2 of keys 2p, 2p+1 over this thread's features
    {   // the head's largest centred magnitudes, for the range guard
        float mk = 0.0f, mv = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int hi = e & 1;
            const float ak = anc[8 * fg + e], av = anc[FD + 8 * fg + e];
            const auto f = [&](uint32_t wd) { return __uint_as_float(hi ? (wd & 0xffff0000u) : (wd << 16)); };
            if (!za) {
                mk = fmaxf(mk, fabsf(f(ka[e >> 1]) - ak));
                mv = fmaxf(mv, fabsf(f(va[e >> 1]) - av));
            }
            if (!zb) {
                mk = fmaxf(mk, fabsf(f(kb[e >> 1]) - ak));
                mv = fmaxf(mv, fabsf(f(vb[e >> 1]) - av));
            }
        }
        mk = wave_max_nonneg(mk);
        mv = wave_max_nonneg(mv);
        if ((tid & 63) == 0) {
            wmax[tid >> 6][0] = mk;
            wmax[tid >> 6][1] = mv;
        }
    }
    float xa[8], xb[8];   // centred fp16 keys 2p, 2p+1 of this thread's features, as floats
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int row = 8 * fg + e;
        const int hi = e & 1;
        const uint32_t kwa = ka[e >> 1], kwb = kb[e >> 1], vwa = va[e >> 1], vwb = vb[e >> 1];
        const float ak = anc[row], av = anc[FD + row];
        h16x2 kk, vv;
        kk[0] = static_cast<_Float16>(za ? 0.0f : __uint_as_float(hi ? (kwa & 0xffff0000u) : (kwa << 16)) - ak);
        kk[1] = static_cast<_Float16>(zb ? 0.0f : __uint_as_float(hi ? (kwb & 0xffff0000u) : (kwb << 16)) - ak);
        vv[0] = static_cast<_Float16>(za ? 0.0f : __uint_as_float(hi ? (vwa & 0xffff0000u) : (vwa << 16)) - av);
        vv[1] = static_cast<_Float16>(zb ? 0.0f : __uint_as_float(hi ? (vwb & 0xffff0000u) : (vwb << 16)) - av);
        dst[row * (M_LD / 2) + pr] = __builtin_bit_cast(uint32_t, kk);
        dst[(FD + row) * (M_LD / 2) + vcol(2 * pr) / 2] = __builtin_bit_cast(uint32_t, vv);
        if (pr < (M_LD - MT) / 2) {   // row padding
            dst[row * (M_LD / 2) + MT / 2 + pr] = 0u;
            dst[(FD + row) * (M_LD / 2) + MT / 2 + pr] = 0u;
        }
        xa[e] = static_cast<float>(kk[0]);
        xb[e] = static_cast<float>(kk[1]);
        vsa = fmaf(static_cast<float>(vv[0]), static_cast<float>(vv[0]), vsa);
        vsb = fmaf(static_cast<float>(vv[1]), static_cast<float>(vv[1]), vsb);
    }
    vpart[fg][2 * pr] = vsa;
    vpart[fg][2 * pr + 1] = vsb;
    // Check image: the 64-point Walsh-Hadamard transform of each key's centred values,
    // X[m] = sum_f (-1)^popcount(f & m) x_f with f = 8 fg + e, m = 8 mh + ml, splits into
    // 8-point transforms over e (here, per thread) and then over fg (below, per key); only
    // odd m (odd ml) are kept: direction t = (m - 1) / 2.
    walsh_transform(xa);
    walsh_transform(xb);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        ys[2 * pr][fg][q4] = xa[2 * q4 + 1];
        ys[2 * pr + 1][fg][q4] = xb[2 * q4 + 1];
    }
    __syncthreads();
    if (tid == 0) {   // the block's range maxima, one atomic each
        float mk = 0.0f, mv = 0.0f;
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
            mk = fmaxf(mk, wmax[w4][0]);
            mv = fmaxf(mv, wmax[w4][1]);
        }
        atomicMax(guard + 1 + 2 * bh, __float_as_uint(mk));
        atomicMax(guard + 2 + 2 * bh, __float_as_uint(mv));
    }
    unsigned char* kut = kuimg + (static_cast<int64_t>(bh) * ntiles + t) * KU_TILE_BYTES;
    {   // thread -> key j, ml = 2 q4 + 1: the 8-point transform over the feature groups
        const int j = tid & (MT - 1), q4 = tid >> 6;
        float x8[8];
#pragma unroll
        for (int g8 = 0; g8 < 8; ++g8) x8[g8] = ys[j][g8][q4];
        walsh_transform(x8);
        _Float16* kur = reinterpret_cast<_Float16*>(kut);
#pragma unroll
        for (int mh = 0; mh < 8; ++mh) kur[(4 * mh + q4) * M_LD + vcol(j)] = static_cast<_Float16>(x8[mh]);
        if (q4 == 0) {
            float nv = 0.0f;
#pragma unroll
            for (int f8 = 0; f8 < 8; ++f8) nv += vpart[f8][j];
            reinterpret_cast<float*>(kut + KU_NRM)[j] = nv;
        }
    }
    if (tid < NCHK) {   // row padding of the projections
        *reinterpret_cast<uint4*>(kut + tid * M_LD * 2 + MT * 2) = make_uint4(0, 0, 0, 0);
    } else if (tid < NCHK + 16) {   // tail after the norms
        *reinterpret_cast<uint4*>(kut + KU_NRM + MT * 4 + (tid - NCHK) * 16) = make_uint4(0, 0, 0, 0);
    }
}

// Score pass with a running max (rows i >= 3d): m_i = max_{j <= i} q_i.k_j / h, in log2
// units.  Block = 4 waves x 2 sets of 16 queries (the sets share the key operands); 64-key
// tiles of the key-major image stream through a ring of three LDS buffers (copied straight
// from the workspace); scores on MFMA (bf16): S^T block kb of a tile, lane (g, c) register
// r = key 16 kb + 4g + r, query c of the set.
__global__ __launch_bounds__(256) void lla_rowmax_kernel(const uint16_t* __restrict__ q,
                                                         const unsigned char* __restrict__ kimg,
                                                         float* __restrict__ mrow, int n, int row0,
                                                         int BH, float sl2) {
    __shared__ __attribute__((aligned(16))) unsigned char ring[3 * KM_TILE_BYTES];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int g = lane >> 4, c = lane & 15;
    const int nrows = n - row0;
    const int nblk = (nrows + R_QB - 1) / R_QB;
    int blk, bh;
    head_major_block(static_cast<int>(blockIdx.x), BH, nblk, &bh, &blk);
    const int q0 = row0 + blk * R_QB;
    const int qlast = min(q0 + R_QB, n) - 1;
    const int wave_first = q0 + wu * R_QW;
    const int wave_last = min(wave_first + R_QW - 1, n - 1);
    const int64_t base = static_cast<int64_t>(bh) * n * FD;
    int qi[R_SETS], qc[R_SETS];   // set st: column c is query wave_first + 16 st + c
    bf16x8 qf[R_SETS][2];
#pragma unroll
    for (int st = 0; st < R_SETS; ++st) {
        qi[st] = wave_first + 16 * st + c;
        qc[st] = min(qi[st], n - 1);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            qf[st][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(
                                                        q + base + static_cast<int64_t>(qc[st]) * FD + ks * 32 + 8 * g));
    }

    const int ntiles = (qlast + MT) / MT;
    const int ptiles = (n + MT - 1) / MT;
    const __amdgpu_buffer_rsrc_t img = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(uniform_ptr(kimg + static_cast<int64_t>(bh) * ptiles * KM_STRIDE)), 0,
        ptiles * KM_STRIDE, 0x00020000);
    int voff[KM_WLOADS];
#pragma unroll
    for (int e = 0; e < KM_WLOADS; ++e) voff[e] = lane * 16 + min(wu + B_WAVES * e, KM_LOADS - 1) * 1024;
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ring));
    // Tile tt -> ring buffer tt % 3; every wave issues KM_WLOADS copies (surplus ones repeat
    // the last chunk); past the last tile the last one is re-read into a dead buffer.
    auto issue = [&](int tt) {
        const int ts = min(tt, ntiles - 1);
        const uint32_t dst = lds0 + static_cast<uint32_t>((tt % 3) * KM_TILE_BYTES);
#pragma unroll
        for (int e = 0; e < KM_WLOADS; ++e) {
            const int u = min(wu + B_WAVES * e, KM_LOADS - 1);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                img, reinterpret_cast<__attribute__((address_space(3))) void*>(static_cast<uintptr_t>(dst + u * 1024)),
                16, voff[e], ts * KM_STRIDE, 0, 0);
        }
    };
    // Only tile copies are in flight in the loop: after tile t+1's come tile t+2's
    // KM_WLOADS, so vmcnt <= KM_WLOADS means tile t+1 has landed.
    auto next_tile = [] {
        __builtin_amdgcn_s_waitcnt(KM_WLOADS | (0x7 << 4) | (0xF << 8));
        LDS_FENCE();
        __builtin_amdgcn_s_barrier();
        LDS_FENCE();
    };

    float m_run[R_SETS];
#pragma unroll
    for (int st = 0; st < R_SETS; ++st) m_run[st] = -INFINITY;
    issue(0);
    issue(1);
    next_tile();
    for (int t = 0; t < ntiles; ++t) {
        issue(t + 2);
        const int j0 = t * MT;
        // Tiles wholly below the wave's first query need no causal mask (a copy without it).
        auto tile_body = [&](auto masked) {
            const unsigned char* cur = ring + (t % 3) * KM_TILE_BYTES;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                bf16x8 a[2];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    a[ks] = __builtin_bit_cast(
                        bf16x8, *reinterpret_cast<const uint4*>(cur + (kb * 16 + c) * (KM_LD * 2) + ks * 64 + 16 * g));
#pragma unroll
                for (int st = 0; st < R_SETS; ++st) {
                    float4v s = {0.f, 0.f, 0.f, 0.f};
                    s = mfma_bf16(a[0], qf[st][0], s);
                    s = mfma_bf16(a[1], qf[st][1], s);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = j0 + kb * 16 + 4 * g + r;
                        m_run[st] = fmaxf(m_run[st], (!decltype(masked)::value || j <= qc[st]) ? s[r] : -INFINITY);
                    }
                }
            }
        };
        if (j0 + MT - 1 <= wave_first) tile_body(std::false_type{});
        else if (j0 <= wave_last) tile_body(std::true_type{});   // wave-uniform
        next_tile();
    }
    // Copies past the last tile are still landing in LDS: let them finish before exit.
    __builtin_amdgcn_s_waitcnt(0x0 | (0x7 << 4) | (0xF << 8));
#pragma unroll
    for (int st = 0; st < R_SETS; ++st) {
        float m = fmaxf(m_run[st], __shfl_xor(m_run[st], 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        if (g == 0 && qi[st] < n) mrow[static_cast<int64_t>(bh) * nrows + (qi[st] - row0)] = m * sl2;
    }
}

// Upper 16x16 block (I, J), I <= J, of a symmetric 64x64 matrix held as 10 MFMA accumulators.
__device__ __forceinline__ constexpr int ublk(int I, int J) { return I * 4 - I * (I - 1) / 2 + (J - I); }

// ---------------------------------------------------------------------------------------
// Rows i >= 3d: the cross moment C_vk is never formed.  Pass 1 (the key-moment blocks) builds
// the key moments and solves for y; pass 2 (lla_probe_kernel) applies C_vk to y in one
// attention-like sweep:
//   b_i = vbar_i - C_vk y_i = a_v + (1/omega') sum_j w_ij t_ij (v_j - a_v),
//   t_ij = 1 + S_k.yh_i / omega' - (k_j - a).yh_i,   yh_i = omega' y_i,
// because the weighted sum of k_j - kbar_i vanishes (the t_ij sum, weighted, to omega').
// Both passes take the weights from bitwise the same score arithmetic.
// x moved within each row of 16 lanes by a DPP pattern (quad_perm, row_mirror, ...).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
constexpr int DPP_QUAD_1032 = 0xB1, DPP_QUAD_2301 = 0x4E, DPP_ROW_HALF_MIRROR = 0x141, DPP_ROW_MIRROR = 0x140;
// Reductions over the 16 lanes of each row (every lane gets its row's result), then over
// the wave through the four row leaders.
__device__ __forceinline__ float row_max_f(float x) {
    x = fmaxf(x, dpp_f<DPP_QUAD_1032>(x));
    x = fmaxf(x, dpp_f<DPP_QUAD_2301>(x));
    x = fmaxf(x, dpp_f<DPP_ROW_HALF_MIRROR>(x));
    return fmaxf(x, dpp_f<DPP_ROW_MIRROR>(x));
}
__device__ __forceinline__ float row_sum_f(float x) {
    x += dpp_f<DPP_QUAD_1032>(x);
    x += dpp_f<DPP_QUAD_2301>(x);
    x += dpp_f<DPP_ROW_HALF_MIRROR>(x);
    return x + dpp_f<DPP_ROW_MIRROR>(x);
}
__device__ __forceinline__ float wave_max_f(float x) {
    x = row_max_f(x);
    return fmaxf(fmaxf(lane_value(x, 0), lane_value(x, 16)), fmaxf(lane_value(x, 32), lane_value(x, 48)));
}
__device__ __forceinline__ float wave_sum_f(float x) {
    x = row_sum_f(x);
    return (lane_value(x, 0) + lane_value(x, 16)) + (lane_value(x, 32) + lane_value(x, 48));
}

constexpr int KQ = 4;                        // queries per wave of pass 1
constexpr int K_BQ = B_WAVES * KQ;           // 16 queries per block: the score MFMA's columns
constexpr int K_IMG = FD * M_LD * 2;         // fp16 key image of a tile (first half of the tile image)
constexpr int K_LOADS = K_IMG / 1024;
constexpr int K_WLOADS = (K_LOADS + B_WAVES - 1) / B_WAVES;
constexpr int K_SW = K_IMG;                  // sqrt-weights [query][key], rows of M_LD halves
constexpr int K_SW2 = K_SW + K_BQ * M_LD * 2;   // fp16 weights, 16 rows (rows >= K_BQ zero)
constexpr int K_BUF = K_SW2 + 16 * M_LD * 2;
// Solve staging, per query: a 64 x 16 float array T[col][t] (a block row of the matrix,
// transposed), its 16-byte chunks XOR-swizzled by bits 1-2 of col so that the 16-byte reads
// and writes of 8 consecutive lanes fall on distinct bank groups.
constexpr int GS_QS = 16 * 68 + 16;          // query stride (floats)
constexpr int K_SOLVE_FLOATS = KQ * GS_QS + KQ * FD;   // per wave: staging + pivots
constexpr int K_SOLVE_BYTES = K_SOLVE_FLOATS * 4 * B_WAVES;
constexpr int K_MEAN_OFF = K_SOLVE_BYTES > M_NBUF * K_BUF ? K_SOLVE_BYTES : M_NBUF * K_BUF;
constexpr int K_SMEM = K_MEAN_OFF + (K_BQ * FD + B_WAVES * 16 + 16) * 4;   // + the check's key scales
constexpr int P_YLD = 2 * FD;                // per query: yh hi (fp16) | yh lo (fp16)
constexpr int P_QSC = 8;                     // per query: gamma, 2^-e, 1/omega', dropped-pivot flag,
                                             // weighted mean |k - a|^2, 3 unused
// Per query, the check's target: the NCHK projections of q - a + lambda e^{-m} y.
constexpr int P_CHK = NCHK;
static_assert(K_IMG % 1024 == 0, "key image must be whole wave copies");
static_assert(K_BQ <= 16, "score MFMA has 16 query columns");

// Lane p of each row of 16 lanes, broadcast to its row (p a compile-time lane).
__device__ __forceinline__ float row_bcast(float x, int p) {
    const int xi = __builtin_bit_cast(int, x);
    int r;
    switch (p) {
        case 0: r = __builtin_amdgcn_update_dpp(0, xi, 0x150, 0xF, 0xF, true); break;
        case 1: r = __builtin_amdgcn_update_dpp(0, xi, 0x151, 0xF, 0xF, true); break;
        case 2: r = __builtin_amdgcn_update_dpp(0, xi, 0x152, 0xF, 0xF, true); break;
        case 3: r = __builtin_amdgcn_update_dpp(0, xi, 0x153, 0xF, 0xF, true); break;
        case 4: r = __builtin_amdgcn_update_dpp(0, xi, 0x154, 0xF, 0xF, true); break;
        case 5: r = __builtin_amdgcn_update_dpp(0, xi, 0x155, 0xF, 0xF, true); break;
        case 6: r = __builtin_amdgcn_update_dpp(0, xi, 0x156, 0xF, 0xF, true); break;
        case 7: r = __builtin_amdgcn_update_dpp(0, xi, 0x157, 0xF, 0xF, true); break;
        case 8: r = __builtin_amdgcn_update_dpp(0, xi, 0x158, 0xF, 0xF, true); break;
        case 9: r = __builtin_amdgcn_update_dpp(0, xi, 0x159, 0xF, 0xF, true); break;
        case 10: r = __builtin_amdgcn_update_dpp(0, xi, 0x15A, 0xF, 0xF, true); break;
        case 11: r = __builtin_amdgcn_update_dpp(0, xi, 0x15B, 0xF, 0xF, true); break;
        case 12: r = __builtin_amdgcn_update_dpp(0, xi, 0x15C, 0xF, 0xF, true); break;
        case 13: r = __builtin_amdgcn_update_dpp(0, xi, 0x15D, 0xF, 0xF, true); break;
        case 14: r = __builtin_amdgcn_update_dpp(0, xi, 0x15E, 0xF, 0xF, true); break;
        default: r = __builtin_amdgcn_update_dpp(0, xi, 0x15F, 0xF, 0xF, true); break;
    }
    return __builtin_bit_cast(float, r);
}

// Solve (C_q + ridge) y_q = z_q for the KQ = 4 queries of a wave at once: LDL^T in 16-column
// panels with the rows of query G on lanes 16 G .. 16 G + 15 (lane 16 G + l holds rows
// l + 16 j, j = 0..3), pivot rows broadcast within each row of 16 lanes.
//   The matrix of query q is C_q - s_q s_q^T / omega'_q + lam[q] I, where
//   ckk[q]: the upper 16x16 blocks of C_q in MFMA accumulator layout (lane (g, c) register r
//           of ckk[q][ublk(I, J)] = entry (16 I + 4 g + r, 16 J + c)); consumed;
//   skq: s of this lane's query (LDS, 64 floats); sks[j] = s[l + 16 j] / omega'.
//   zr[j]: right-hand side of row l + 16 j of this lane's query (updated).
//   thr: pivots <= thr are dropped, their unknowns set to zero.
//   Sg: this wave's LDS area of K_SOLVE_FLOATS floats.
// Panel K is staged from the accumulators to the row layout through LDS, eliminated there,
// and its multipliers go back through LDS as MFMA operands for the trailing update
// C_IJ -= L_IK D_K L_JK^T (fp32 16x16x4 MFMAs, per query) of the blocks still in the
// accumulators; the multipliers stay in registers for the back substitution, which forms
// each y_P as x_P minus a row-of-16 reduction.  Returns y in yr[j].
// Offset (floats) of chunk tc (entries 4 tc .. 4 tc + 3) of column col in a query's staging.
__device__ __forceinline__ int gs_chunk(int col, int tc) { return col * 16 + ((tc ^ ((col >> 1) & 3)) << 2); }

// Panel K of group_solve (a template, so that every register index is a constant).
template <int K>
__device__ __forceinline__ void group_panel(float4v (&ckk)[KQ][10], float (&zr)[4], const float thr,
                                            const float (&lam)[KQ], const float (&sks)[4], const float* skq,
                                            float* Sg, float (&Lk)[4][4][16], float (&dk)[4], const int g,
                                            const int c) {
    const int G = g, l = c;   // row layout: query G, row offset l
    float* Dg = Sg + KQ * GS_QS;
    // Block row K of every query, ridge on the diagonal, transposed: T_q[col][t] =
    // C_q[16 K + t][col]; lane (g, c) holds t = 4g .. 4g + 3 of column 16 J + c, one chunk.
#pragma unroll
    for (int q = 0; q < KQ; ++q)
#pragma unroll
        for (int J = K; J < 4; ++J) {
            float4v val = ckk[q][ublk(K, J)];
            if (J == K) {
#pragma unroll
                for (int r = 0; r < 4; ++r) val[r] += 4 * g + r == c ? lam[q] : 0.0f;
            }
            *reinterpret_cast<float4v*>(Sg + q * GS_QS + gs_chunk(16 * J + c, g)) = val;
        }
    LDS_FENCE();
    // Panel rows of this lane's query: Lf[j][t] = C[16 K + t][l + 16 j] = C[l + 16 j][16 K + t].
    float Lf[4][16];
#pragma unroll
    for (int j = K; j < 4; ++j)
#pragma unroll
        for (int tc = 0; tc < 4; ++tc) {
            const float4v x = *reinterpret_cast<const float4v*>(Sg + G * GS_QS + gs_chunk(16 * j + l, tc));
#pragma unroll
            for (int r = 0; r < 4; ++r) Lf[j][4 * tc + r] = x[r];
        }
    LDS_FENCE();
    // Rank-one downdate, applied to each entry once, as its panel is staged (the trailing
    // updates are linear, so it commutes with them): C -= S_k S_k^T / omega'.
    float skt[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) skt[t] = skq[16 * K + t];
#pragma unroll
    for (int j = K; j < 4; ++j)
#pragma unroll
        for (int t = 0; t < 16; ++t) Lf[j][t] = fmaf(-sks[j], skt[t], Lf[j][t]);
    float d = 0.0f;
#pragma unroll
    for (int p = 0; p < 16; ++p) {
        const float piv = row_bcast(Lf[K][p], p);
        // Reciprocal pivot (about 1 ulp); a dropped pivot gets a zero column of L.
        const float inv = piv > thr ? __builtin_amdgcn_rcpf(piv) : 0.0f;
        int row = l;
        asm volatile("" : "+v"(row));   // row tests per step: no precomputed lane masks
        float f[4];
#pragma unroll
        for (int j = K + 1; j < 4; ++j) f[j] = Lf[j][p] * inv;
        f[K] = row > p ? Lf[K][p] * inv : 0.0f;
        const float zp = row_bcast(zr[K], p);
#pragma unroll
        for (int j = K; j < 4; ++j) zr[j] = fmaf(-f[j], zp, zr[j]);
#pragma unroll
        for (int t = p + 1; t < 16; ++t) {
            const float bt = row_bcast(Lf[K][t], p);
#pragma unroll
            for (int j = K; j < 4; ++j) Lf[j][t] = fmaf(-f[j], bt, Lf[j][t]);
        }
        d = row == p ? piv : d;
#pragma unroll
        for (int j = K; j < 4; ++j) Lf[j][p] = f[j];
    }
    dk[K] = d;
#pragma unroll
    for (int j = K; j < 4; ++j)
#pragma unroll
        for (int t = 0; t < 16; ++t) Lk[K][j][t] = Lf[j][t];
    if (K < 3) {
        // Multipliers of the later blocks' rows (transposed as above: T[l + 16 j][t] =
        // L[l + 16 j][16 K + t]) and the pivots, read back per query as MFMA operands over
        // the panel columns 16 K + 4 g + s (K-slot g of step s: one chunk per operand).
#pragma unroll
        for (int j = K + 1; j < 4; ++j)
#pragma unroll
            for (int tc = 0; tc < 4; ++tc)
                *reinterpret_cast<float4v*>(Sg + G * GS_QS + gs_chunk(16 * j + l, tc)) =
                    float4v{Lf[j][4 * tc], Lf[j][4 * tc + 1], Lf[j][4 * tc + 2], Lf[j][4 * tc + 3]};
        Dg[G * FD + 16 * K + l] = d;
        LDS_FENCE();
#pragma unroll
        for (int q = 0; q < KQ; ++q) {
            float dv[4], Lo[4][4];
            const float4v dq = *reinterpret_cast<const float4v*>(Dg + q * FD + 16 * K + 4 * g);
#pragma unroll
            for (int X = K + 1; X < 4; ++X) {
                const float4v x = *reinterpret_cast<const float4v*>(Sg + q * GS_QS + gs_chunk(16 * X + c, g));
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) Lo[X][s4] = x[s4];
            }
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) dv[s4] = dq[s4];
#pragma unroll
            for (int I = K + 1; I < 4; ++I)
#pragma unroll
                for (int J = I; J < 4; ++J)
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4)
                        ckk[q][ublk(I, J)] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                            -Lo[I][s4], dv[s4] * Lo[J][s4], ckk[q][ublk(I, J)], 0, 0, 0);
        }
        LDS_FENCE();
    }
}

__device__ __forceinline__ void group_solve(float4v (&ckk)[KQ][10], float (&zr)[4], const float thr,
                                            const float (&lam)[KQ], const float (&sks)[4], const float* skq,
                                            float* Sg, float (&yr)[4], const int g, const int c, float& dropped) {
    float Lk[4][4][16];       // Lk[K][j][t] = L[l + 16 j][16 K + t], j >= K
    float dk[4];              // pivot of row l + 16 K
    group_panel<0>(ckk, zr, thr, lam, sks, skq, Sg, Lk, dk, g, c);
    group_panel<1>(ckk, zr, thr, lam, sks, skq, Sg, Lk, dk, g, c);
    group_panel<2>(ckk, zr, thr, lam, sks, skq, Sg, Lk, dk, g, c);
    group_panel<3>(ckk, zr, thr, lam, sks, skq, Sg, Lk, dk, g, c);
    const int l = c;
    // Back substitution L^T y = x, x = D^{-1} z (zero at dropped pivots), from the last row:
    // y_P = x_P - sum_{b > P} L[b][P] y_b, the sum over this query's 16 lanes.  L[b][P] is
    // zero for rows b <= P of the diagonal block, and y of rows not yet solved is zero.
    float x[4];
    float drop = 0.0f;   // 1 if a pivot of this lane's rows was dropped
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float inv_d = __builtin_amdgcn_rcpf(dk[j]);
        inv_d = fmaf(inv_d, fmaf(-dk[j], inv_d, 1.0f), inv_d);   // one Newton step: ~0.5 ulp
        x[j] = dk[j] > thr ? zr[j] * inv_d : 0.0f;
        drop = dk[j] > thr ? drop : 1.0f;
        yr[j] = 0.0f;
    }
    dropped = row_max_f(drop);   // over the query's 16 lanes
#pragma unroll
    for (int P = FD - 1; P >= 0; --P) {
        const int jP = P / 16, p = P % 16;
        float part = 0.0f;
#pragma unroll
        for (int j = jP; j < 4; ++j) part = fmaf(Lk[jP][j][p], yr[j], part);
        const float sum = row_sum_f(part);
        int row = l;
        asm volatile("" : "+v"(row));
        yr[jP] = row == p ? x[jP] - sum : yr[jP];
    }
}

// Pass 1.  Block = 4 waves x KQ queries = 16 consecutive queries; wave w owns queries
// i0 + w + 4 qq (interleaved, so the causal tail splits evenly).  Per 64-key tile: scores of
// key block w for all 16 queries (one bf16 MFMA pair), sqrt-weights and fp16 weights to LDS;
// per 32-key half, each wave forms R = sqrt(w) (k - a) for its queries from the shared fp16
// key image (one rounding) and accumulates C_kk = sum R R^T (10 upper blocks per query), and
// the block sums S_k = sum w (k - a) of all 16 queries (one MFMA, features 16w..).  Then per
// query: (C_kk - S_k S_k^T / omega' + lambda e^{-m} I) y = kbar - q, kbar = a + S_k / omega',
// and the scaled solution yh 2^e = omega' y 2^e in [2^13, 2^14) goes out as fp16 hi + lo
// parts with gamma = 1 + S_k.yh / omega'.
__device__ __forceinline__ void keymom_block(
    const int bidx, unsigned char* smem, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const float* __restrict__ mrow, const float* __restrict__ anchors, const unsigned char* __restrict__ packed,
    _Float16* __restrict__ yhl, float* __restrict__ qsc, float* __restrict__ chk,
    const unsigned* __restrict__ guard, int n, int row0, int rowp, int BH, float sl2, float lambda) {

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int g = lane >> 4, c = lane & 15;
    const int nrows = n - row0;   // rows of the row-max array
    const int prows = n - rowp;   // rows of this path
    const int nblk = (prows + K_BQ - 1) / K_BQ;
    int blk, bh;
    head_major_block(bidx, BH, nblk, &bh, &blk);

    const int i0 = rowp + blk * K_BQ;
    const int last = min(i0 + K_BQ - 1, n - 1);
    const int64_t base = static_cast<int64_t>(bh) * n * FD;
    const uint16_t* kh = k + base;
    if (head_unsafe(guard, bh)) return;   // block-uniform: the probe pass hands the rows back

    if (K_BQ < 16) {   // rows K_BQ.. of every Sw2 buffer: the zero rows of the weight operand
        for (int e = tid; e < M_NBUF * (16 - K_BQ) * M_LD / 8; e += 256) {
            const int bsel = e / ((16 - K_BQ) * M_LD / 8), rem = e % ((16 - K_BQ) * M_LD / 8);
            *reinterpret_cast<uint4*>(smem + bsel * K_BUF + K_SW2 + K_BQ * M_LD * 2 + rem * 16) =
                make_uint4(0, 0, 0, 0);
        }
    }
    // Score operand: column c < K_BQ is query i0 + c.
    const int qcol = min(i0 + c, n - 1);
    const bool colv = c < K_BQ;
    const float mcol = mrow[static_cast<int64_t>(bh) * nrows + (qcol - row0)];   // log2 units
    bf16x8 qf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (colv) raw = *reinterpret_cast<const uint4*>(q + base + static_cast<int64_t>(qcol) * FD + ks * 32 + 8 * g);
        qf[ks] = __builtin_bit_cast(bf16x8, raw);
    }

    // Scores of key block w (16 keys) of a tile: lane (g, c) register r = query c, key
    // 16w + 4g + r.  Issued before the tile's moments, stored after.  om2p sums the fp16
    // weights of query c over this lane's keys.
    float om2p = 0.0f;
    const float hs = 0.5f * sl2, hm = 0.5f * mcol;
    auto score_mfma = [&](uint4 kq0, uint4 kq1) {
        float4v s = {0.f, 0.f, 0.f, 0.f};
        s = mfma_bf16(__builtin_bit_cast(bf16x8, kq0), qf[0], s);
        return mfma_bf16(__builtin_bit_cast(bf16x8, kq1), qf[1], s);
    };
    auto score_store = [&](float4v s, unsigned char* buf, int j0) {
        float e[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) e[rr] = __builtin_amdgcn_exp2f(fmaf(s[rr], hs, -hm));
        if (j0 + MT - 1 > i0) {   // block-uniform: keys past some query of the block
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) e[rr] = j0 + 16 * w + 4 * g + rr <= qcol ? e[rr] : 0.0f;
        }
        half4 sw4;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) sw4[rr] = static_cast<_Float16>(e[rr]);
        const half4 w4 = sw4 * sw4;
        if (colv) {
            *reinterpret_cast<half4*>(reinterpret_cast<_Float16*>(buf + K_SW) + c * M_LD + 16 * w + 4 * g) = sw4;
            *reinterpret_cast<half4*>(reinterpret_cast<_Float16*>(buf + K_SW2) + c * M_LD + 16 * w + 4 * g) = w4;
            const h16x2 one = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
            om2p = __builtin_amdgcn_fdot2(__builtin_shufflevector(w4, w4, 0, 1), one, om2p, false);
            om2p = __builtin_amdgcn_fdot2(__builtin_shufflevector(w4, w4, 2, 3), one, om2p, false);
        }
    };

    float4v ckk[KQ][10];
#pragma unroll
    for (int qq = 0; qq < KQ; ++qq)
#pragma unroll
        for (int t = 0; t < 10; ++t) ckk[qq][t] = float4v{0.f, 0.f, 0.f, 0.f};
    // S_k of the block's queries: lane (g, c) register r = query 4g + r, feature 16w + c.
    float4v sk = {0.f, 0.f, 0.f, 0.f};

    const int ntiles = (last + MT) / MT;
    const int ptiles = (n + MT - 1) / MT;
    // The key half of the head's tile images, copied straight into LDS (wave w takes KiB
    // chunks w, w+4, w+8; every wave issues exactly K_WLOADS copies, surplus ones repeating
    // the last chunk).  Score operand (key 16w + c, bf16) read through a buffer resource whose
    // size ends at key n, so keys past n read as zero.
    const __amdgpu_buffer_rsrc_t img = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(uniform_ptr(packed + static_cast<int64_t>(bh) * ptiles * PACK_TILE_BYTES)),
        0, ptiles * PACK_TILE_BYTES, 0x00020000);
    int voff[K_WLOADS];
#pragma unroll
    for (int e = 0; e < K_WLOADS; ++e) voff[e] = lane * 16 + min(wu + B_WAVES * e, K_LOADS - 1) * 1024;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(uniform_ptr(reinterpret_cast<const unsigned char*>(kh))), 0, n * FD * 2,
        0x00020000);
    const int kq_off = (16 * w + c) * FD * 2 + 16 * g;
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem));
    auto buf = [&](int tt) { return smem + (tt % M_NBUF) * K_BUF; };
    // Tile tt: its score operand first, then its image, so that waiting for the operand
    // (vector loads complete in issue order) does not also wait for the copies.
    auto issue = [&](int tt, uint4& q0, uint4& q1) {
        const int ts = min(tt, ntiles - 1);
        const uint32_t dst = lds0 + static_cast<uint32_t>((tt % M_NBUF) * K_BUF);
        q0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(krs, kq_off, ts * MT * FD * 2, 0));
        q1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(krs, kq_off + 64, ts * MT * FD * 2, 0));
#pragma unroll
        for (int e = 0; e < K_WLOADS; ++e) {
            const int u = min(wu + B_WAVES * e, K_LOADS - 1);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                img, reinterpret_cast<__attribute__((address_space(3))) void*>(static_cast<uintptr_t>(dst + u * 1024)),
                16, voff[e], ts * PACK_TILE_BYTES, 0, 0);
        }
    };
    // After tile t+1's copies come tile t+2's 2 + K_WLOADS loads.
    static_assert(K_WLOADS + 2 < 16, "vmcnt operand is 4 bits here");
    auto wait_tile = [] {
        __builtin_amdgcn_s_waitcnt((K_WLOADS + 2) | (0x7 << 4) | (0xF << 8));
        LDS_FENCE();
    };
    auto ring_barrier = [] {
        __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
        LDS_FENCE();
        __builtin_amdgcn_s_barrier();
        LDS_FENCE();
    };
    auto compute = [&](int t, const unsigned char* cur, int sub) {
        const int j0 = t * MT;
        const _Float16* Kt = reinterpret_cast<const _Float16*>(cur);
        const _Float16* Sw = reinterpret_cast<const _Float16*>(cur + K_SW);
        const _Float16* Sw2 = reinterpret_cast<const _Float16*>(cur + K_SW2);
        {
            if (j0 + 32 * sub > last) return;   // block-uniform: past every query of the block
            const int ko = 32 * sub + 8 * g;
            half8 kf[4];
#pragma unroll
            for (int fb = 0; fb < 4; ++fb) kf[fb] = *reinterpret_cast<const half8*>(Kt + (fb * 16 + c) * M_LD + ko);
            const half8 w8 = *reinterpret_cast<const half8*>(Sw2 + c * M_LD + ko);
            const half8 kw = *reinterpret_cast<const half8*>(Kt + (wu * 16 + c) * M_LD + ko);   // = kf[w]
            // Every query of the wave takes the whole half-tile: keys past a query carry
            // weight zero, so one straight-line block lets loads, forming and MFMAs overlap.
#pragma unroll
            for (int qq = 0; qq < KQ; ++qq) {
                const half8 sw = *reinterpret_cast<const half8*>(Sw + (wu + 4 * qq) * M_LD + ko);
                half8 rk[4];
#pragma unroll
                for (int fb = 0; fb < 4; ++fb) rk[fb] = kf[fb] * sw;
                int idx = 0;
#pragma unroll
                for (int fb = 0; fb < 4; ++fb)
#pragma unroll
                    for (int fb2 = fb; fb2 < 4; ++fb2) {
                        ckk[qq][idx] = mfma_f16(rk[fb], rk[fb2], ckk[qq][idx]);
                        ++idx;
                    }
            }
            sk = mfma_f16(w8, kw, sk);
        }
    };
    // Step t: tile t in LDS, tile t+1's image landing and its score operand (issued a step
    // ago) in B, tile t+2 issued now into A; tile t+1's scores are taken between the halves.
    uint4 aq0, aq1, bq0, bq1;
    issue(0, aq0, aq1);
    issue(1, bq0, bq1);
    wait_tile();
    score_store(score_mfma(aq0, aq1), buf(0), 0);
    ring_barrier();
    for (int t = 0; t < ntiles; t += 2) {
        issue(t + 2, aq0, aq1);
        compute(t, buf(t), 0);
        const float4v sb = score_mfma(bq0, bq1);
        compute(t, buf(t), 1);
        if (t + 1 < ntiles) score_store(sb, buf(t + 1), (t + 1) * MT);
        wait_tile();
        ring_barrier();
        if (t + 1 >= ntiles) break;
        issue(t + 3, bq0, bq1);
        compute(t + 1, buf(t + 1), 0);
        const float4v sa = score_mfma(aq0, aq1);
        compute(t + 1, buf(t + 1), 1);
        if (t + 2 < ntiles) score_store(sa, buf(t + 2), (t + 2) * MT);
        wait_tile();
        ring_barrier();
    }
    // Copies issued past the last tile may still be landing in ring buffers that the solve
    // area overlaps: wait for this wave's loads (the barrier below covers the others).
    __builtin_amdgcn_s_waitcnt(0x0 | (0x7 << 4) | (0xF << 8));
    LDS_FENCE();

    // ---- block sums -> LDS (outside the solve area)
    float* skm = reinterpret_cast<float*>(smem + K_MEAN_OFF);   // [query][feature]
    float* omp = skm + K_BQ * FD;                                // [wave][query]
    om2p += __shfl_xor(om2p, 16);
    om2p += __shfl_xor(om2p, 32);
#pragma unroll
    for (int r = 0; r < 4; ++r)
        if (4 * g + r < K_BQ) skm[(4 * g + r) * FD + 16 * w + c] = sk[r];
    if (g == 0 && colv) omp[w * 16 + c] = om2p;
    __syncthreads();

    // ---- the 4 solves at once; row layout: lane 16 G + l holds rows l + 16 j of query
    // i0 + wu + 4 G (a query past n is solved but not stored).  z = kbar - q with
    // kbar = a + S_k / omega'.
    float* Sg = reinterpret_cast<float*>(smem) + w * K_SOLVE_FLOATS;
    const float* anc = anchors + static_cast<int64_t>(bh) * 2 * FD;
    float lam_q[KQ];
#pragma unroll
    for (int qq = 0; qq < KQ; ++qq) {
        const int iq = min(i0 + wu + 4 * qq, n - 1);
        lam_q[qq] = lambda * exp2f(-mrow[static_cast<int64_t>(bh) * nrows + (iq - row0)]);
    }
    const int G = g, l = c;
    const int qlG = wu + 4 * G;
    const int iqG = i0 + qlG;
    const int iqc = min(iqG, n - 1);
    float om2 = 0.0f;
#pragma unroll
    for (int t = 0; t < B_WAVES; ++t) om2 += omp[t * 16 + qlG];
    const float iom2 = 1.0f / om2;   // >= 1: the query's top-scoring key has weight 1
    const float* mqG = skm + qlG * FD;
    float zr[4], sks[4], yr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int a = l + 16 * j;
        const float skv = mqG[a];
        sks[j] = skv * iom2;
        zr[j] = fmaf(skv, iom2, anc[a]) - bf16_bits_to_f32(q[base + static_cast<int64_t>(iqc) * FD + a]);
    }
    // lambda > 0: drop only pivots that rounding made non-positive; lambda = 0: also drop
    // directions the prefix leaves (numerically) undetermined, below 1e-6 of the largest
    // diagonal entry of the (downdated) matrix.
    float thr = 0.0f;
    if (!(lambda > 0.0f)) {
        float dm[KQ];
#pragma unroll
        for (int qq = 0; qq < KQ; ++qq) {
            const float* mq = skm + (wu + 4 * qq) * FD;
            float oq = 0.0f;
#pragma unroll
            for (int t = 0; t < B_WAVES; ++t) oq += omp[t * 16 + wu + 4 * qq];
            float dmax = -INFINITY;
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (4 * g + r == c) {
                        const float sv = mq[16 * I + c];
                        dmax = fmaxf(dmax, ckk[qq][ublk(I, I)][r] - sv * sv / oq + lam_q[qq]);
                    }
            dm[qq] = wave_max_f(dmax);
        }
        thr = 1e-6f * (G == 0 ? dm[0] : G == 1 ? dm[1] : G == 2 ? dm[2] : dm[3]);
    }
    // The check's key scale: trace of sum R R^T (before the downdate) / omega', the weighted
    // mean of |k - a|^2.
    float trq[KQ];
#pragma unroll
    for (int qq = 0; qq < KQ; ++qq) {
        float tr = 0.0f;
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int r = 0; r < 4; ++r) tr += 4 * g + r == c ? ckk[qq][ublk(I, I)][r] : 0.0f;
        trq[qq] = wave_sum_f(tr);
    }
    // Values needed after the solve go through LDS or are derived again there, so that
    // nothing but the solve's own state is live across it.
    float* trs = omp + B_WAVES * 16;   // [query] the check's key scale
    if (lane == 0) {
#pragma unroll
        for (int qq = 0; qq < KQ; ++qq) trs[wu + 4 * qq] = trq[qq];
    }
    float dropped = 0.0f;
    group_solve(ckk, zr, thr, lam_q, sks, mqG, Sg, yr, g, c, dropped);
    const float trG = trs[qlG];
    const float lamG = lambda * exp2f(-mrow[static_cast<int64_t>(bh) * nrows + (iqc - row0)]);
    // Check target: the LLA weights reproduce linear functions of the keys, so applied to the
    // centred keys they give q - a + lambda e^{-m} y (exactly, for the y they were formed
    // with); projected on the NCHK directions, direction t at feature f = l + 16 j carrying
    // the sign (-1)^popcount(f & (2t + 1)).
    float cv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int a = l + 16 * j;
        cv[j] = bf16_bits_to_f32(q[base + static_cast<int64_t>(iqc) * FD + a]) - anc[a] + lamG * yr[j];
    }
    float chk_lo = 0.0f, chk_hi = 0.0f;   // directions l and l + 16
#pragma unroll
    for (int tq = 0; tq < NCHK; ++tq) {
        const int m = 2 * tq + 1;
        const bool sl = (__builtin_popcount(l & (m & 15)) & 1) != 0;
        float part = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool sj = (__builtin_popcount(j & (m >> 4)) & 1) != 0;
            part += (sl != sj) ? -cv[j] : cv[j];
        }
        const float sum = row_sum_f(part);
        if (tq < 16) chk_lo = l == tq ? sum : chk_lo;
        else chk_hi = l == tq - 16 ? sum : chk_hi;
    }
    // yh 2^e with max |.| in [2^13, 2^14), as fp16 hi + lo (about 22 bits together), and
    // gamma = 1 + S_k . yh / omega'.
    float yh[4], amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        yh[j] = yr[j] * om2;
        amax = fmaxf(amax, fabsf(yh[j]));
    }
    amax = row_max_f(amax);
    int ex = 0;
    (void)frexpf(amax, &ex);
    ex = max(ex, -100);   // keeps 2^(14 - ex) finite
    const float sig = amax > 0.0f ? ldexpf(1.0f, 14 - ex) : 1.0f;
    _Float16 hi[4], lo[4];
    float dot = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float ys = yh[j] * sig;
        hi[j] = static_cast<_Float16>(ys);
        lo[j] = static_cast<_Float16>(ys - static_cast<float>(hi[j]));
        dot = fmaf(mqG[l + 16 * j], static_cast<float>(hi[j]) + static_cast<float>(lo[j]), dot);
    }
    dot = row_sum_f(dot);
    if (iqG < n) {
        const int64_t qrow = static_cast<int64_t>(bh) * prows + (iqG - rowp);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            yhl[qrow * P_YLD + l + 16 * j] = hi[j];
            yhl[qrow * P_YLD + FD + l + 16 * j] = lo[j];
        }
        // qsc[3] flags a pivot dropped although the ridge keeps the system positive definite.
        if (l == 0) {
            *reinterpret_cast<float4v*>(qsc + qrow * P_QSC) =
                float4v{fmaf(dot / sig, iom2, 1.0f), 1.0f / sig, iom2, lambda > 0.0f ? dropped : 0.0f};
            *reinterpret_cast<float4v*>(qsc + qrow * P_QSC + 4) = float4v{trG * iom2, 0.0f, 0.0f, 0.0f};
        }
        chk[qrow * P_CHK + l] = chk_lo;
        chk[qrow * P_CHK + 16 + l] = chk_hi;
    }
}

// Pass 2.  Block = 4 waves x 32 queries (two sets of 16 per wave, which share the key and
// value operands), two blocks per CU; each 64-key tile (bf16 keys and fp16 centred keys, both
// key-major, and fp16 centred values feature-major) is copied into one of two LDS buffers
// while the other is in use.  Per tile,
// wave and query set, for key block kb (16 keys):
//   S^T = K Q^T (bf16 MFMA pair: pass 1's operands in pass 1's order, so bitwise its scores),
//   U^T = (K - a) (yh_hi + yh_lo)^T 2^e (four fp16 MFMAs),
//   P = fp16(w fp16(gamma - U 2^-e)) with w = fp16(sqrt-weight)^2 as in pass 1 (packed fp16);
// lane (g, c) register r holds key 16 kb + 4g + r of query c, which is already the A
// operand of O += P (V - a_v) over 32-key steps (K-slots: keys 4g.., then 16 + 4g..), and
// of the check sums OK += P (projected K - a), with sum w |v - a_v|^2 on the side.
//   The check: the LLA weights l_j = P_j / omega' reproduce the centred query,
// sum_j l_j (k_j - a) = q - a + lambda e^{-m} y, for the y the weights were formed with and
// the moments of the same rounded data; the fp16 factor R of pass 1 breaks that identity by
// as much as its rounding moves y.  The projected deviation, in units of the weighted rms of
// |k - a| and scaled by the weighted rms of |v - a_v| over |b|, tracks the row's relative
// error; rows above CHK_TOL go to the fp64 kernel.
constexpr int P_WAVES = 4;
constexpr int P_NBUF = 2;
constexpr int P_SETS = 2;                    // query sets of 16 per wave
constexpr int P_QW = 16 * P_SETS;
constexpr int P_QB = P_WAVES * P_QW;
constexpr int P_BUF = 2 * KM_TILE_BYTES + FD * M_LD * 2 + KU_TILE_BYTES;   // bf16 K | fp16 K - a | fp16 V - a_v | check image
constexpr int P_LOADS = P_BUF / 1024;
constexpr int P_WLOADS = (P_LOADS + P_WAVES - 1) / P_WAVES;
constexpr int P_SMEM = P_NBUF * P_BUF;
static_assert(P_BUF % 1024 == 0 && 2 * KM_TILE_BYTES % 1024 == 0, "probe images must be whole wave copies");

__global__ __launch_bounds__(P_WAVES * 64, 2) void lla_probe_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ mrow, const float* __restrict__ anchors,
    const unsigned char* __restrict__ packed, const unsigned char* __restrict__ kimg,
    const unsigned char* __restrict__ kuimg, const _Float16* __restrict__ yhl, const float* __restrict__ qsc,
    const float* __restrict__ chk, float* __restrict__ out, unsigned* __restrict__ guard, int* __restrict__ list,
    int n, int row0, int rowp, int BH, float sl2) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int g = lane >> 4, c = lane & 15;
    const int nrows = n - row0, prows = n - rowp;
    const int nblk = (prows + P_QB - 1) / P_QB;
    int blk, bh;
    head_major_block(static_cast<int>(blockIdx.x), BH, nblk, &bh, &blk);
    const int i0 = rowp + blk * P_QB;
    const int qw0 = i0 + P_QW * wu;                   // this wave's first query
    const int wave_last = min(qw0 + P_QW - 1, n - 1);
    const int block_last = min(i0 + P_QB - 1, n - 1);
    const int64_t base = static_cast<int64_t>(bh) * n * FD;
    if (head_unsafe(guard, bh)) {   // block-uniform: the head's rows go to the fp64 kernel
#pragma unroll
        for (int st = 0; st < P_SETS; ++st)
            if (g == 0 && qw0 + 16 * st + c < n) hand_back(guard, list, bh, n, qw0 + 16 * st + c);
        return;
    }

    // Query set st: column c is query qw0 + 16 st + c (clamped to n - 1).
    bf16x8 qf[P_SETS][2];
    half8 yh[P_SETS][2], yl[P_SETS][2];
    float gam[P_SETS], isig[P_SETS], hm[P_SETS];
    int qc[P_SETS];
#pragma unroll
    for (int st = 0; st < P_SETS; ++st) {
        qc[st] = min(qw0 + 16 * st + c, n - 1);
        const int64_t qrow = static_cast<int64_t>(bh) * prows + (qc[st] - rowp);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            qf[st][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(
                                                        q + base + static_cast<int64_t>(qc[st]) * FD + 32 * ks + 8 * g));
            yh[st][ks] = *reinterpret_cast<const half8*>(yhl + qrow * P_YLD + 32 * ks + 8 * g);
            yl[st][ks] = *reinterpret_cast<const half8*>(yhl + qrow * P_YLD + FD + 32 * ks + 8 * g);
        }
        const float4v sc = *reinterpret_cast<const float4v*>(qsc + qrow * P_QSC);
        gam[st] = sc[0];
        isig[st] = sc[1];
        hm[st] = 0.5f * mrow[static_cast<int64_t>(bh) * nrows + (qc[st] - row0)];
    }
    const float hs = 0.5f * sl2;

    const int ntiles = block_last / MT + 1;
    const int ptiles = (n + MT - 1) / MT;
    const __amdgpu_buffer_rsrc_t kres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(uniform_ptr(kimg + static_cast<int64_t>(bh) * ptiles * KM_STRIDE)), 0,
        ptiles * KM_STRIDE, 0x00020000);
    const __amdgpu_buffer_rsrc_t vres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(uniform_ptr(packed + static_cast<int64_t>(bh) * ptiles * PACK_TILE_BYTES)), 0,
        ptiles * PACK_TILE_BYTES, 0x00020000);
    const __amdgpu_buffer_rsrc_t ures = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(uniform_ptr(kuimg + static_cast<int64_t>(bh) * ptiles * KU_TILE_BYTES)), 0,
        ptiles * KU_TILE_BYTES, 0x00020000);
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem));
    // Chunk u of a buffer: u < 18 from the key-major images, u < 27 from the value half of the
    // tile image, the rest from the check image.  Wave w issues chunks w, w+4, ..., w+28.
    constexpr int U_KM = 2 * KM_TILE_BYTES / 1024, U_V = U_KM + FD * M_LD * 2 / 1024;
    auto issue = [&](int tt) {
        const int ts = min(tt, ntiles - 1);
        const uint32_t dst = lds0 + static_cast<uint32_t>((tt % P_NBUF) * P_BUF);
#pragma unroll
        for (int e = 0; e < P_WLOADS; ++e) {
            const int u = min(wu + P_WAVES * e, P_LOADS - 1);
            auto* ldst = reinterpret_cast<__attribute__((address_space(3))) void*>(static_cast<uintptr_t>(dst + u * 1024));
            if (u < U_KM)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(kres, ldst, 16, lane * 16 + u * 1024, ts * KM_STRIDE, 0, 0);
            else if (u < U_V)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(vres, ldst, 16, lane * 16 + K_IMG + (u - U_KM) * 1024,
                                                         ts * PACK_TILE_BYTES, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ures, ldst, 16, lane * 16 + (u - U_V) * 1024,
                                                         ts * KU_TILE_BYTES, 0, 0);
        }
    };
    // The copies of the next tile have landed (all loads waited for) and every wave is done
    // with the buffer they will overwrite next.
    auto wait_and_sync = [] {
        __builtin_amdgcn_s_waitcnt(0x0 | (0x7 << 4) | (0x0 << 8));
        LDS_FENCE();
        __builtin_amdgcn_s_barrier();
        LDS_FENCE();
    };

    float4v o[P_SETS][4], ok[P_SETS][NCHK / 16];
    float wvn[P_SETS];   // sum w |v - a_v|^2 of query c over this lane's keys
#pragma unroll
    for (int st = 0; st < P_SETS; ++st) {
#pragma unroll
        for (int fv = 0; fv < 4; ++fv) o[st][fv] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < NCHK / 16; ++db) ok[st][db] = float4v{0.f, 0.f, 0.f, 0.f};
        wvn[st] = 0.0f;
    }
    issue(0);
    wait_and_sync();
    // A tile wholly below the wave's first query needs no causal mask: those tiles (all but
    // the last one or two of a wave) run first, in a loop of their own with the unmasked
    // body, so the accumulators keep one register assignment from tile to tile.
    auto tile_step = [&](const int t, auto phase) {
        issue(t + 1);   // into the buffer tile t-1 used
        const int j0 = t * MT;
        auto tile_body = [&](auto masked) {
            const unsigned char* cur = smem + (t % P_NBUF) * P_BUF;
            const unsigned char* KB = cur;
            const unsigned char* KC = cur + KM_TILE_BYTES;
            const _Float16* VI = reinterpret_cast<const _Float16*>(cur + 2 * KM_TILE_BYTES);
            const _Float16* UI = reinterpret_cast<const _Float16*>(cur + 2 * KM_TILE_BYTES + FD * M_LD * 2);
            const float* NR = reinterpret_cast<const float*>(cur + 2 * KM_TILE_BYTES + FD * M_LD * 2 + KU_NRM);
            half4 p[P_SETS][4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int ro = (kb * 16 + c) * (KM_LD * 2) + 16 * g;
                const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(KB + ro);
                const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(KB + ro + 64);
                const half8 c0 = *reinterpret_cast<const half8*>(KC + ro);
                const half8 c1 = *reinterpret_cast<const half8*>(KC + ro + 64);
#pragma unroll
                for (int st = 0; st < P_SETS; ++st) {
                    float4v sv = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
                    sv = mfma_bf16(k0, qf[st][0], sv);
                    sv = mfma_bf16(k1, qf[st][1], sv);
                    u = mfma_f16(c0, yh[st][0], u);
                    u = mfma_f16(c1, yh[st][1], u);
                    u = mfma_f16(c0, yl[st][0], u);
                    u = mfma_f16(c1, yl[st][1], u);
                    const bool full = !decltype(masked)::value || j0 + MT - 1 <= qw0 + 16 * st;
                    half4 sw4, t4;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float e = __builtin_amdgcn_exp2f(fmaf(sv[r], hs, -hm[st]));
                        if (!full) e = j0 + kb * 16 + 4 * g + r <= qc[st] ? e : 0.0f;
                        sw4[r] = static_cast<_Float16>(e);
                        t4[r] = static_cast<_Float16>(fmaf(-u[r], isig[st], gam[st]));
                    }
                    const half4 w4 = sw4 * sw4;   // w = fp16(sw^2) exactly as pass 1
                    p[st][kb] = w4 * t4;          // P = fp16(w t)
                    const float4v nr = *reinterpret_cast<const float4v*>(NR + kb * 16 + 4 * g);
#pragma unroll
                    for (int r = 0; r < 4; ++r) wvn[st] = fmaf(static_cast<float>(w4[r]), nr[r], wvn[st]);
                }
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int fv = 0; fv < 4; ++fv) {
                    const half8 vb = *reinterpret_cast<const half8*>(VI + (fv * 16 + c) * M_LD + 32 * ks + 8 * g);
#pragma unroll
                    for (int st = 0; st < P_SETS; ++st) {
                        const half8 pa = __builtin_shufflevector(p[st][2 * ks], p[st][2 * ks + 1], 0, 1, 2, 3, 4, 5, 6, 7);
                        o[st][fv] = mfma_f16(pa, vb, o[st][fv]);
                    }
                }
#pragma unroll
                for (int db = 0; db < NCHK / 16; ++db) {
                    const half8 ub = *reinterpret_cast<const half8*>(UI + (db * 16 + c) * M_LD + 32 * ks + 8 * g);
#pragma unroll
                    for (int st = 0; st < P_SETS; ++st) {
                        const half8 pa = __builtin_shufflevector(p[st][2 * ks], p[st][2 * ks + 1], 0, 1, 2, 3, 4, 5, 6, 7);
                        ok[st][db] = mfma_f16(pa, ub, ok[st][db]);
                    }
                }
            }
        };
        if constexpr (!decltype(phase)::value) tile_body(std::false_type{});
        else if (j0 <= wave_last) tile_body(std::true_type{});   // wave-uniform
        wait_and_sync();
    };
    const int tfull = min(ntiles, (qw0 + 1) / MT);   // tiles t with t MT + MT - 1 <= qw0
    for (int t = 0; t < tfull; ++t) tile_step(t, std::false_type{});
    for (int t = tfull; t < ntiles; ++t) tile_step(t, std::true_type{});
    // Copies issued past the last tile are still landing in LDS: let them finish before exit.
    __builtin_amdgcn_s_waitcnt(0x0 | (0x7 << 4) | (0xF << 8));

    // Output rows: lane (g, c) register r of set st = query qw0 + 16 st + 4g + r, feature 16 fv + c
    // (direction 16 db + c of the check sums).  A row goes to the fp64 kernel if its output is
    // not finite, its solve dropped a pivot (qsc[3]), or its check exceeds CHK_TOL.
    const float* anc = anchors + static_cast<int64_t>(bh) * 2 * FD + FD;
#pragma unroll
    for (int st = 0; st < P_SETS; ++st) {
        // sum_j w_j |v_j - a_v|^2 of query c (over all keys), then of query 4g + r below
        float vq = wvn[st];
        vq += __shfl_xor(vq, 16);
        vq += __shfl_xor(vq, 32);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = qw0 + 16 * st + 4 * g + r;
            const int64_t qrow = static_cast<int64_t>(bh) * prows + (min(i, n - 1) - rowp);
            const float4v sc = *reinterpret_cast<const float4v*>(qsc + qrow * P_QSC);
            const float kn2 = qsc[qrow * P_QSC + 4];
            float bb = 0.0f, rr = 0.0f;
#pragma unroll
            for (int fv = 0; fv < 4; ++fv) {
                const float ov = fmaf(o[st][fv][r], sc[2], anc[fv * 16 + c]);
                bb = fmaf(ov, ov, bb);
                if (i < n) out[base + static_cast<int64_t>(i) * FD + fv * 16 + c] = ov;
            }
#pragma unroll
            for (int db = 0; db < NCHK / 16; ++db) {
                const float dv = fmaf(ok[st][db][r], sc[2], -chk[qrow * P_CHK + 16 * db + c]);
                rr = fmaf(dv, dv, rr);
            }
            bb = row_sum_f(bb);
            rr = row_sum_f(rr);
            const float vn2 = __shfl(vq, 4 * g + r) * sc[2];
            // (|res| / |k - a|_rms)^2 (|v - a_v|_rms / |b|)^2 against CHK_TOL^2; NaN fails.
            const float est2 = (rr * (1.0f / NCHK)) * vn2 / (kn2 * bb);
            const bool bad = i < n && (!(est2 <= CHK_TOL * CHK_TOL) || sc[3] != 0.0f);
            const uint64_t badm = __ballot(bad);   // every lane takes part
            if (c == 0 && i < n && ((badm >> (16 * g)) & 0xFFFFull) != 0) hand_back(guard, list, bh, n, i);
        }
    }
}

// ---------------------------------------------------------------------------------------
// Rows i < 3d of the bf16 path, in fp64: one wave per row, 4 consecutive rows per block
// sharing the (at most 3d-key) prefix staged in LDS as bf16.
//   scores -> m, weights, omega; kbar, vbar (lane = feature);
//   C_kk = R^T R with R[j] = sqrt(w_j) (k_j - kbar) in fp64 on the matrix cores
//   (v_mfma_f64_16x16x4f64, 4 keys per step), ridge on the diagonal, then moved to
//   lane-per-row form through LDS, 16 rows at a time;
//   LDL^T elimination lane-per-row, back substitution -> y;
//   probe u_j = (k_j - kbar).y and b = vbar - sum_j w_j u_j (v_j - vbar)  (= vbar - C_vk y).
// fp64 MFMA output layout: D[4 r + (l / 16)][l % 16] in double register r of lane l.
constexpr int S_ROWS = 4;
constexpr int S_KMAX = 3 * FD;
constexpr int S_KPL = S_KMAX / 64;   // keys per lane in the score and probe passes
constexpr int S_KLD = FD + 2;   // bf16 row stride (halves): 33 words, conflict-free per row
constexpr int S_TLD = FD + 1;   // fp64 row stride of the transposition buffer

typedef double double4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double wave_max_d(double x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmax(x, __shfl_xor(x, off));
    return x;
}
__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

// LDS of a short-row block: staged K, V (bf16), then per wave q, weights, kbar, and 8 rows of
// C_kk in transit (fp64), whose first FD entries then serve as the pivot-row exchange (then y).
constexpr int SB_KS = 0;
constexpr int SB_VS = SB_KS + S_KMAX * S_KLD * 2;
constexpr int SB_QS = SB_VS + S_KMAX * S_KLD * 2;
constexpr int SB_WS = SB_QS + S_ROWS * FD * 8;
constexpr int SB_KBS = SB_WS + S_ROWS * S_KMAX * 8;
constexpr int SB_VBS = SB_KBS + S_ROWS * FD * 8;           // vbar (held in LDS across the solve)
constexpr int SB_TB = SB_VBS + S_ROWS * FD * 8;
constexpr int S_SMEM = SB_TB + S_ROWS * 8 * S_TLD * 8;
static_assert(2 * (S_SMEM > K_SMEM ? S_SMEM : K_SMEM) <= 160 * 1024, "two blocks per CU");
static_assert(SB_QS % 16 == 0, "fp64 areas stay aligned");

__device__ __forceinline__ void short_block(
    const int bidx, unsigned char* smem, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, float* __restrict__ out, int n, int rows, int BH,
    double inv_h, double lambda) {
    uint16_t* Ks = reinterpret_cast<uint16_t*>(smem + SB_KS);
    uint16_t* Vs = reinterpret_cast<uint16_t*>(smem + SB_VS);
    double (*qs)[FD] = reinterpret_cast<double (*)[FD]>(smem + SB_QS);
    double (*ws)[S_KMAX] = reinterpret_cast<double (*)[S_KMAX]>(smem + SB_WS);
    double (*kbs)[FD] = reinterpret_cast<double (*)[FD]>(smem + SB_KBS);
    double (*vbs)[FD] = reinterpret_cast<double (*)[FD]>(smem + SB_VBS);
    double (*tb)[8 * S_TLD] = reinterpret_cast<double (*)[8 * S_TLD]>(smem + SB_TB);   // 8 rows of C_kk in transit

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int nblk = (rows + S_ROWS - 1) / S_ROWS;
    const int blk = nblk - 1 - bidx / BH;  // longest rows first
    const int bh = bidx % BH;
    const int r0 = blk * S_ROWS;
    const int i = r0 + w;
    const bool valid = i < rows;
    const int ic = min(i, rows - 1);
    const int nk = min(r0 + S_ROWS, rows);          // keys staged: 0 .. nk-1
    const int64_t base = static_cast<int64_t>(bh) * n * FD;
    auto kval = [&](int j, int a) { return static_cast<double>(bf16_bits_to_f32(Ks[j * S_KLD + a])); };
    auto vval = [&](int j, int a) { return static_cast<double>(bf16_bits_to_f32(Vs[j * S_KLD + a])); };

    for (int e = tid; e < nk * (FD / 2); e += 256) {   // 32-bit words: 2 features
        const int j = e / (FD / 2), f0 = (e % (FD / 2)) * 2;
        *reinterpret_cast<uint32_t*>(Ks + j * S_KLD + f0) =
            *reinterpret_cast<const uint32_t*>(k + base + static_cast<int64_t>(j) * FD + f0);
        *reinterpret_cast<uint32_t*>(Vs + j * S_KLD + f0) =
            *reinterpret_cast<const uint32_t*>(v + base + static_cast<int64_t>(j) * FD + f0);
    }
    qs[w][lane] = static_cast<double>(bf16_bits_to_f32(q[base + static_cast<int64_t>(ic) * FD + lane]));
    __syncthreads();

    // ---- scores of keys lane + 64 h, running max, weights, omega
    double s[S_KPL];
#pragma unroll
    for (int h2 = 0; h2 < S_KPL; ++h2) {
        s[h2] = -INFINITY;
        const int j = lane + 64 * h2;
        if (j <= ic) {
            double acc = 0.0;
#pragma unroll 16
            for (int a = 0; a < FD; ++a) acc = fma(qs[w][a], kval(j, a), acc);
            s[h2] = acc * inv_h;
        }
    }
    double smax = s[0];
#pragma unroll
    for (int h2 = 1; h2 < S_KPL; ++h2) smax = fmax(smax, s[h2]);
    const double m = wave_max_d(smax);
    double wsum = 0.0;
#pragma unroll
    for (int h2 = 0; h2 < S_KPL; ++h2) {
        const double wj = (lane + 64 * h2 <= ic) ? exp(s[h2] - m) : 0.0;
        ws[w][lane + 64 * h2] = wj;
        wsum += wj;
    }
    const double omega = wave_sum_d(wsum);
    LDS_FENCE();

    // ---- weighted means, lane = feature
    double ka = 0.0, va = 0.0;
    for (int j = 0; j <= ic; ++j) {
        const double wj = ws[w][j];
        ka = fma(wj, kval(j, lane), ka);
        va = fma(wj, vval(j, lane), va);
    }
    ka /= omega;
    va /= omega;
    kbs[w][lane] = ka;
    vbs[w][lane] = va;
    LDS_FENCE();

    // ---- C_kk on the matrix cores: upper 16x16 blocks (I, J), I <= J, 4 keys per step.
    double kb4[4];
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) kb4[fb] = kbs[w][16 * fb + c];
    double4v cacc[10];
#pragma unroll
    for (int t = 0; t < 10; ++t) cacc[t] = double4v{0.0, 0.0, 0.0, 0.0};
    const int nsteps = (ic + 4) / 4;
    for (int st = 0; st < nsteps; ++st) {
        const int j = 4 * st + g;          // this lane's key (K-slot g)
        const bool in = j <= ic;
        const double sw = in ? sqrt(ws[w][j]) : 0.0;
        double a4[4];
#pragma unroll
        for (int fb = 0; fb < 4; ++fb) a4[fb] = in ? sw * (kval(j, 16 * fb + c) - kb4[fb]) : 0.0;
        int idx = 0;
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int J = I; J < 4; ++J) {
                cacc[idx] = __builtin_amdgcn_mfma_f64_16x16x4f64(a4[I], a4[J], cacc[idx], 0, 0, 0);
                ++idx;
            }
    }
    // ridge on the diagonal (row 4r + g of a diagonal block equals column c), its maximum
    const double lam_s = lambda * exp(-m);
    double dmax = 0.0;
    {
        int idx = 0;
#pragma unroll
        for (int I = 0; I < 4; ++I) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (4 * r + g == c) {
                    cacc[idx][r] += lam_s;
                    dmax = fmax(dmax, cacc[idx][r]);
                }
            idx += 4 - I;
        }
    }
    dmax = wave_max_d(dmax);
    const double thresh = lambda > 0.0 ? 0.0 : 1e-12 * dmax;

    // ---- to lane-per-row form: pass pp stages rows 8 pp .. 8 pp + 7 (half hh of block row
    // P = pp / 2) and lanes 8 pp .. read them
    double cr[FD];
    double* T = tb[w];
#pragma unroll
    for (int pp = 0; pp < 8; ++pp) {
        const int P = pp / 2, hh = pp % 2;
        int idx = 0;
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int J = I; J < 4; ++J) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    // block (I, J), register r: C[16I + 4r + g][16J + c]
                    if (I == P) {
                        if (r / 2 == hh) T[(4 * (r - 2 * hh) + g) * S_TLD + 16 * J + c] = cacc[idx][r];
                    } else if (J == P) {
                        if (c / 8 == hh) T[(c - 8 * hh) * S_TLD + 16 * I + 4 * r + g] = cacc[idx][r];
                    }
                }
                ++idx;
            }
        LDS_FENCE();
        if (lane / 8 == pp) {
#pragma unroll
            for (int b = 0; b < FD; ++b) cr[b] = T[(lane % 8) * S_TLD + b];
        }
        LDS_FENCE();
    }
    double z = ka - qs[w][lane];

    // ---- LDL^T elimination (lane owns row), then back substitution
    double* xw = T;   // the transposition buffer, no longer needed, holds the pivot row
#pragma unroll
    for (int p = 0; p < FD; ++p) {
        xw[lane] = cr[p];
        LDS_FENCE();
        const double piv = xw[p];
        const double inv = piv > thresh ? 1.0 / piv : 0.0;
        const double f = lane > p ? cr[p] * inv : 0.0;
        const double zp = __shfl(z, p);
        z = fma(-f, zp, z);
#pragma unroll
        for (int b = p + 1; b < FD; ++b) cr[b] = fma(-f, xw[b], cr[b]);
        LDS_FENCE();
    }
    double ylane = 0.0;
#pragma unroll
    for (int p = FD - 1; p >= 0; --p) {
        const double dp = __shfl(cr[p], p);
        const double zp = __shfl(z, p);
        const double yp = dp > thresh ? zp / dp : 0.0;
        ylane = lane == p ? yp : ylane;
        z = fma(-cr[p], yp, z);
    }
    xw[lane] = ylane;
    LDS_FENCE();

    // ---- probe: u_j = (k_j - kbar).y for keys lane + 64 h; then b = vbar - C_vk y
    double wusum = 0.0;
#pragma unroll
    for (int h2 = 0; h2 < S_KPL; ++h2) {
        const int j = lane + 64 * h2;
        double wu = 0.0;
        if (j <= ic) {
            double u = 0.0;
#pragma unroll 16
            for (int a = 0; a < FD; ++a) u = fma(kval(j, a) - kbs[w][a], xw[a], u);
            wu = ws[w][j] * u;   // this lane's own weight entry, overwritten just below
        }
        ws[w][j] = wu;
        wusum += wu;
    }
    const double swu = wave_sum_d(wusum);
    LDS_FENCE();
    double acc = 0.0;
    for (int j = 0; j <= ic; ++j) acc = fma(ws[w][j], vval(j, lane), acc);
    const double vb = vbs[w][lane];
    if (valid) out[base + static_cast<int64_t>(i) * FD + lane] = static_cast<float>(vb - (acc - vb * swu));
}

// Rows handed back by the range guard and the checks, in fp64: one wave per listed row, its
// prefix streamed through LDS 64 keys at a time (scores recomputed in each pass), with the
// arithmetic of the short rows: weights e^{s - m}, kbar and vbar (lane = feature), C_kk about
// kbar on the matrix cores (v_mfma_f64_16x16x4f64), lane-per-row LDL^T, and
// b = vbar - C_vk y through u_j = (k_j - kbar).y.  Any prefix length; the wave's latency
// scales with the prefix, not with a block-wide elimination.
constexpr int RF_WAVES = 4;
constexpr int RF_KLD = FD + 2;    // bf16 row stride (halves) of a staged chunk: 33 words
struct RefineWave {
    double qs[FD];                // the query
    double ws[MT];                // per-chunk weights (then w_j u_j)
    double kb[FD];                // kbar
    double xb[FD];                // pivot-row exchange, then y
    double tb[16 * S_TLD];        // 16 rows of C_kk in transit
    uint16_t ks[MT * RF_KLD];     // staged keys
    uint16_t vs[MT * RF_KLD];     // staged values
};

__global__ __launch_bounds__(RF_WAVES * 64) void lla_refine_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    float* __restrict__ out, const int* __restrict__ list, const unsigned* __restrict__ count, int n,
    double inv_h, double lambda) {
    __shared__ RefineWave lds[RF_WAVES];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int g = lane >> 4, c = lane & 15;
    RefineWave& L = lds[w];
    const int total = static_cast<int>(*count);
    for (int e = static_cast<int>(blockIdx.x) * RF_WAVES + w; e < total;
         e += static_cast<int>(gridDim.x) * RF_WAVES) {
        const int code = list[e];
        const int bh = code / n, i = code % n, cnt = i + 1;
        const int64_t base = static_cast<int64_t>(bh) * n * FD;
        const uint16_t* kh = k + base;
        const uint16_t* vh = v + base;
        L.qs[lane] = static_cast<double>(bf16_bits_to_f32(q[base + static_cast<int64_t>(i) * FD + lane]));
        // Stage keys (and values) c0 .. c0 + 63 of the prefix, zero past it: lane j copies
        // row c0 + j (8 x 16 bytes).
        auto stage = [&](int c0, bool with_v) {
            const int j = c0 + lane;
#pragma unroll
            for (int u = 0; u < FD / 8; ++u) {
                uint4 kx = make_uint4(0, 0, 0, 0), vx = kx;
                if (j < cnt) {
                    kx = *reinterpret_cast<const uint4*>(kh + static_cast<int64_t>(j) * FD + 8 * u);
                    if (with_v) vx = *reinterpret_cast<const uint4*>(vh + static_cast<int64_t>(j) * FD + 8 * u);
                }
                const uint32_t kw[4] = {kx.x, kx.y, kx.z, kx.w}, vw[4] = {vx.x, vx.y, vx.z, vx.w};
#pragma unroll
                for (int h2 = 0; h2 < 4; ++h2) {
                    *reinterpret_cast<uint32_t*>(L.ks + lane * RF_KLD + 8 * u + 2 * h2) = kw[h2];
                    if (with_v) *reinterpret_cast<uint32_t*>(L.vs + lane * RF_KLD + 8 * u + 2 * h2) = vw[h2];
                }
            }
            LDS_FENCE();
        };
        auto kval = [&](int jj, int a) { return static_cast<double>(bf16_bits_to_f32(L.ks[jj * RF_KLD + a])); };
        auto vval = [&](int jj, int a) { return static_cast<double>(bf16_bits_to_f32(L.vs[jj * RF_KLD + a])); };
        auto score = [&](int jj) {   // staged key jj (this lane's), scaled by 1/h
            double acc = 0.0;
#pragma unroll 16
            for (int a = 0; a < FD; ++a) acc = fma(L.qs[a], kval(jj, a), acc);
            return acc * inv_h;
        };
        LDS_FENCE();

        // ---- pass 1: the row maximum of the scores
        double mloc = -INFINITY;
        for (int c0 = 0; c0 < cnt; c0 += MT) {
            stage(c0, false);
            if (c0 + lane < cnt) mloc = fmax(mloc, score(lane));
            LDS_FENCE();
        }
        const double m = wave_max_d(mloc);

        // ---- pass 2: omega, kbar, vbar (lane = feature)
        double om = 0.0, ka = 0.0, va = 0.0;
        for (int c0 = 0; c0 < cnt; c0 += MT) {
            stage(c0, true);
            const double wj = c0 + lane < cnt ? exp(score(lane) - m) : 0.0;
            L.ws[lane] = wj;
            om += wj;
            LDS_FENCE();
            const int nk = min(MT, cnt - c0);
            for (int jj = 0; jj < nk; ++jj) {
                const double wv = L.ws[jj];
                ka = fma(wv, kval(jj, lane), ka);
                va = fma(wv, vval(jj, lane), va);
            }
            LDS_FENCE();
        }
        om = wave_sum_d(om);
        ka /= om;
        va /= om;
        L.kb[lane] = ka;
        LDS_FENCE();

        // ---- pass 3: C_kk = R^T R, R[j] = sqrt(w_j) (k_j - kbar), upper 16x16 blocks, 4 keys a step
        double kb4[4];
#pragma unroll
        for (int fb = 0; fb < 4; ++fb) kb4[fb] = L.kb[16 * fb + c];
        double4v cacc[10];
#pragma unroll
        for (int t = 0; t < 10; ++t) cacc[t] = double4v{0.0, 0.0, 0.0, 0.0};
        for (int c0 = 0; c0 < cnt; c0 += MT) {
            stage(c0, false);
            L.ws[lane] = c0 + lane < cnt ? exp(score(lane) - m) : 0.0;
            LDS_FENCE();
            const int nk = min(MT, cnt - c0);
            for (int st = 0; st < (nk + 3) / 4; ++st) {
                const int jj = 4 * st + g;
                const bool in = jj < nk;
                const double sw = in ? sqrt(L.ws[jj]) : 0.0;
                double a4[4];
#pragma unroll
                for (int fb = 0; fb < 4; ++fb) a4[fb] = in ? sw * (kval(jj, 16 * fb + c) - kb4[fb]) : 0.0;
                int idx = 0;
#pragma unroll
                for (int I = 0; I < 4; ++I)
#pragma unroll
                    for (int J = I; J < 4; ++J) {
                        cacc[idx] = __builtin_amdgcn_mfma_f64_16x16x4f64(a4[I], a4[J], cacc[idx], 0, 0, 0);
                        ++idx;
                    }
            }
            LDS_FENCE();
        }
        // ridge on the diagonal, its largest entry
        const double lam_s = lambda * exp(-m);
        double dmax = 0.0;
        {
            int idx = 0;
#pragma unroll
            for (int I = 0; I < 4; ++I) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (4 * r + g == c) {
                        cacc[idx][r] += lam_s;
                        dmax = fmax(dmax, cacc[idx][r]);
                    }
                idx += 4 - I;
            }
        }
        dmax = wave_max_d(dmax);
        const double thresh = lambda > 0.0 ? 0.0 : 1e-12 * dmax;

        // ---- to lane-per-row form through LDS, 16 rows at a time
        double cr[FD];
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
            int idx = 0;
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int J = I; J < 4; ++J) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if (I == pp) L.tb[(4 * r + g) * S_TLD + 16 * J + c] = cacc[idx][r];
                        else if (J == pp) L.tb[c * S_TLD + 16 * I + 4 * r + g] = cacc[idx][r];
                    }
                    ++idx;
                }
            LDS_FENCE();
            if (g == pp) {
#pragma unroll
                for (int b = 0; b < FD; ++b) cr[b] = L.tb[c * S_TLD + b];
            }
            LDS_FENCE();
        }
        double z = ka - L.qs[lane];

        // ---- LDL^T elimination (lane owns row), back substitution
#pragma unroll
        for (int pp = 0; pp < FD; ++pp) {
            L.xb[lane] = cr[pp];
            LDS_FENCE();
            const double piv = L.xb[pp];
            const double inv = piv > thresh ? 1.0 / piv : 0.0;
            const double f = lane > pp ? cr[pp] * inv : 0.0;
            const double zp = __shfl(z, pp);
            z = fma(-f, zp, z);
#pragma unroll
            for (int b = pp + 1; b < FD; ++b) cr[b] = fma(-f, L.xb[b], cr[b]);
            LDS_FENCE();
        }
        double ylane = 0.0;
#pragma unroll
        for (int pp = FD - 1; pp >= 0; --pp) {
            const double dp = __shfl(cr[pp], pp);
            const double zp = __shfl(z, pp);
            const double yp = dp > thresh ? zp / dp : 0.0;
            ylane = lane == pp ? yp : ylane;
            z = fma(-cr[pp], yp, z);
        }
        L.xb[lane] = ylane;
        LDS_FENCE();

        // ---- pass 4: u_j = (k_j - kbar).y, then b = vbar - C_vk y
        double swu = 0.0, acc = 0.0;
        for (int c0 = 0; c0 < cnt; c0 += MT) {
            stage(c0, true);
            double wu = 0.0;
            if (c0 + lane < cnt) {
                double u = 0.0;
#pragma unroll 16
                for (int a = 0; a < FD; ++a) u = fma(kval(lane, a) - L.kb[a], L.xb[a], u);
                wu = exp(score(lane) - m) * u;
            }
            L.ws[lane] = wu;
            swu += wu;
            LDS_FENCE();
            const int nk = min(MT, cnt - c0);
            for (int jj = 0; jj < nk; ++jj) acc = fma(L.ws[jj], vval(jj, lane), acc);
            LDS_FENCE();
        }
        swu = wave_sum_d(swu);
        out[base + static_cast<int64_t>(i) * FD + lane] = static_cast<float>(va - (acc - va * swu));
    }
}

// All row work after the row maxima in one launch: short rows (fp64) and the key-moment
// blocks of rows >= 3d.  The short blocks (the "aux" blocks) fill every other run of R_CHUNK
// dispatch positions at the start, so that a CU tends to hold one aux block, mostly
// latency-bound, beside a key-moment block, mostly on the matrix cores (the dispatcher places
// blocks b and b + CU count together).
struct RowsArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* mrow;
    const float* anchors;
    const unsigned char* packed;
    _Float16* yhl;
    float* qsc;
    float* chk;
    float* out;
    unsigned* guard;   // range maxima and the count of rows handed back to the fp64 kernel
    int* list;         // rows handed back
    int n, row0, rowp, BH, n_short, n_key;
    float sl2, lambda;
    double inv_h, lambda_d;
};
constexpr int R_CHUNK = 256;

// Dispatch position b -> key-moment block *key or aux block *aux (the other one -1): runs of
// up to R_CHUNK key-moment blocks and R_CHUNK aux blocks alternate, key-moment first, while
// both kinds remain; then the rest of whichever kind is left.  A bijection from
// [0, n_key + n_aux); a position past that range gets neither role.
__device__ __forceinline__ void rows_block_role(int b, int n_key, int n_aux, int* key, int* aux) {
    const int both = min(n_key, n_aux) / R_CHUNK;   // full rounds of one run of each kind
    if (b < 2 * both * R_CHUNK) {
        const int r = b / (2 * R_CHUNK), o = b % (2 * R_CHUNK);
        if (o < R_CHUNK) *key = r * R_CHUNK + o;
        else *aux = r * R_CHUNK + o - R_CHUNK;
        return;
    }
    b -= 2 * both * R_CHUNK;
    const int kr = n_key - both * R_CHUNK, ar = n_aux - both * R_CHUNK;   // left of each kind
    const int kc = min(R_CHUNK, kr);   // one more (partial) key-moment run, then the aux left,
    if (b < kc) { *key = both * R_CHUNK + b; return; }   // then the key-moment blocks left
    b -= kc;
    if (b < ar) { *aux = both * R_CHUNK + b; return; }
    b -= ar;
    if (b < kr - kc) *key = both * R_CHUNK + kc + b;
}
constexpr int R_SMEM = K_SMEM > S_SMEM ? K_SMEM : S_SMEM;

__global__ __launch_bounds__(256, 2) void lla_rows_kernel(const RowsArgs a) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    int aux = -1, key = -1;
    rows_block_role(static_cast<int>(blockIdx.x), a.n_key, a.n_short, &key, &aux);
    if (aux >= 0) {
        short_block(aux, smem, a.q, a.k, a.v, a.out, a.n, a.row0, a.BH, a.inv_h, a.lambda_d);
    } else if (key >= 0) {
        keymom_block(key, smem, a.q, a.k, a.mrow, a.anchors, a.packed, a.yhl, a.qsc, a.chk, a.guard, a.n, a.row0,
                     a.rowp, a.BH, a.sl2, a.lambda);
    }
}

// Rows [0, 3d): fp64 short-row blocks; [3d, n): key moments and probe pass.
int fast_row0(int64_t n, int64_t d) { return static_cast<int>(n < 3 * d ? n : 3 * d); }

// Fast-path workspace, each region 256-byte aligned:
//   row maxima [B*H][n - 3d] | anchor partial sums [B*H][16][2d] | anchors [B*H][2d] |
//   key/value tile images [B*H][tiles] | key-major key images (bf16, centred fp16)
//   [B*H][tiles] | check images [B*H][tiles] | probe solutions (fp16 hi, lo) [B*H][n - 3d][2d] |
//   probe scalars [B*H][n - 3d][8] | check targets [B*H][n - 3d][32] | guard: count of rows
//   handed back, then per head the largest |k - a| and |v - a_v| (float bits) [1 + 2 B*H] |
//   rows handed back [B*H][n - 3d].
struct FastLayout {
    int64_t mrow, partial, anchors, packed, kimg, kuimg, yhl, qsc, chk, guard, list, total;
};

FastLayout fast_layout(int64_t BH, int64_t n, int64_t d) {
    auto up = [](int64_t bytes) { return (bytes + 255) & ~int64_t(255); };
    const int64_t rows = n - fast_row0(n, d), prows = rows, tiles = (n + MT - 1) / MT;
    FastLayout L;
    L.mrow = 0;
    L.partial = L.mrow + up(BH * rows * 4);
    L.anchors = L.partial + up(BH * ANCHOR_SLICES * 2 * d * 4);
    L.packed = L.anchors + up(BH * 2 * d * 4);
    L.kimg = L.packed + BH * tiles * PACK_TILE_BYTES;
    L.kuimg = L.kimg + BH * tiles * KM_STRIDE;
    L.yhl = L.kuimg + BH * tiles * KU_TILE_BYTES;
    L.qsc = L.yhl + up(BH * prows * P_YLD * 2);
    L.chk = L.qsc + up(BH * prows * P_QSC * 4);
    L.guard = L.chk + up(BH * prows * P_CHK * 4);
    L.list = L.guard + up((1 + 2 * BH) * 4);
    L.total = L.list + up(BH * rows * 4);
    return L;
}

}  // namespace

bool fast_supports(int dtype, int64_t d, int64_t n) {
    // Buffer resources address a head's keys and tile images with 32-bit byte offsets.
    return dtype == 1 && ((d == FD && n <= kFastMaxN) || (d == 128 && n <= kFast128MaxN));
}

size_t fast_workspace_bytes(int64_t B, int64_t H, int64_t n, int64_t d) {
    if (d == 128) return fast128_workspace_bytes(B, H, n);
    if (n - fast_row0(n, d) <= 0) return 0;
    return static_cast<size_t>(fast_layout(B * H, n, d).total);
}

int64_t fast_fallback_count_offset(int64_t B, int64_t H, int64_t n, int64_t d) {
    if (d == 128) return fast128_fallback_count_offset(B, H, n);
    if (n - fast_row0(n, d) <= 0) return -1;
    return fast_layout(B * H, n, d).guard;
}

namespace {
// Dynamic-LDS limits are set per device, the first time a device launches this path.
std::mutex g_attr_mu;
bool g_attr_done[64] = {};

hipError_t ensure_attributes() {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_attr_mu);
    if (g_attr_done[dev]) return hipSuccess;
    if ((err = hipFuncSetAttribute(reinterpret_cast<const void*>(&lla_rows_kernel),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, R_SMEM)) != hipSuccess)
        return err;
    if ((err = hipFuncSetAttribute(reinterpret_cast<const void*>(&lla_probe_kernel),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, P_SMEM)) != hipSuccess)
        return err;
    g_attr_done[dev] = true;
    return hipSuccess;
}
}  // namespace

hipError_t launch_fast(const Problem& p, void* workspace) {
    if (p.d == 128) return launch_fast128(p, workspace);
    hipError_t attr_err = ensure_attributes();
    if (attr_err != hipSuccess) return attr_err;

    const int n = static_cast<int>(p.n);
    const int BH = static_cast<int>(p.B * p.H);
    const int row0 = fast_row0(p.n, p.d);
    const int rowp = row0;   // the key-moment and probe passes start where the short rows end
    const float sl2 = static_cast<float>(LOG2E / p.h);
    const auto* q = static_cast<const uint16_t*>(p.q);
    const auto* k = static_cast<const uint16_t*>(p.k);
    const auto* v = static_cast<const uint16_t*>(p.v);
    RowsArgs ra{};
    ra.q = q; ra.k = k; ra.v = v; ra.out = p.out;
    ra.n = n; ra.row0 = row0; ra.rowp = rowp; ra.BH = BH;
    ra.sl2 = sl2; ra.lambda = static_cast<float>(p.lambda);
    ra.inv_h = 1.0 / p.h; ra.lambda_d = p.lambda;
    ra.n_short = BH * ((row0 + S_ROWS - 1) / S_ROWS);
    const int n_key = n > rowp ? BH * ((n - rowp + K_BQ - 1) / K_BQ) : 0;
    ra.n_key = n_key;
    hipError_t err;
    const unsigned char* kimg_c = nullptr;
    const unsigned char* kuimg_c = nullptr;
    if (n > row0) {
        const FastLayout L = fast_layout(BH, n, p.d);
        unsigned char* ws = static_cast<unsigned char*>(workspace);
        float* mrow = reinterpret_cast<float*>(ws + L.mrow);
        float* partial = reinterpret_cast<float*>(ws + L.partial);
        float* anchors = reinterpret_cast<float*>(ws + L.anchors);
        unsigned char* packed = ws + L.packed;
        unsigned char* kimg = ws + L.kimg;
        kimg_c = kimg;
        ra.mrow = mrow; ra.anchors = anchors; ra.packed = packed;
        ra.yhl = reinterpret_cast<_Float16*>(ws + L.yhl);
        ra.qsc = reinterpret_cast<float*>(ws + L.qsc);
        ra.guard = reinterpret_cast<unsigned*>(ws + L.guard);
        ra.chk = reinterpret_cast<float*>(ws + L.chk);
        kuimg_c = ws + L.kuimg;
        ra.list = reinterpret_cast<int*>(ws + L.list);
        const int ptiles = (n + MT - 1) / MT;
        prof_begin(p.stream, "lla_anchor_kernel");
        lla_anchor_kernel<<<dim3(static_cast<unsigned>(BH) * ANCHOR_SLICES), dim3(256), 0, p.stream>>>(
            k, v, partial, ra.guard, n);
        prof_end(p.stream);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        prof_begin(p.stream, "lla_pack_kernel");
        lla_pack_kernel<<<dim3(static_cast<unsigned>(BH) * ptiles), dim3(256), 0, p.stream>>>(
            k, v, partial, anchors, packed, kimg, ws + L.kuimg, ra.guard, n, ptiles);
        prof_end(p.stream);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        const unsigned blocks_a = static_cast<unsigned>(BH) * ((n - row0 + R_QB - 1) / R_QB);
        prof_begin(p.stream, "lla_rowmax_kernel");
        lla_rowmax_kernel<<<dim3(blocks_a), dim3(256), 0, p.stream>>>(q, kimg, mrow, n, row0, BH, sl2);
        prof_end(p.stream);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    prof_begin(p.stream, "lla_rows_kernel");
    lla_rows_kernel<<<dim3(static_cast<unsigned>(ra.n_short + n_key)), dim3(256), R_SMEM, p.stream>>>(ra);
    prof_end(p.stream);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (n_key > 0) {
        const unsigned blocks_p = static_cast<unsigned>(BH) * ((n - rowp + P_QB - 1) / P_QB);
        prof_begin(p.stream, "lla_probe_kernel");
        lla_probe_kernel<<<dim3(blocks_p), dim3(P_WAVES * 64), P_SMEM, p.stream>>>(
            q, ra.mrow, ra.anchors, ra.packed, kimg_c, kuimg_c, ra.yhl, ra.qsc, ra.chk, p.out, ra.guard, ra.list, n,
            row0, rowp, BH, sl2);
        prof_end(p.stream);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (n > row0) {   // rows handed back by the range guard and the checks, in fp64
        const int cap = BH * (n - row0);
        const int waves = cap < 4096 ? cap : 4096;
        prof_begin(p.stream, "lla_refine_kernel");
        lla_refine_kernel<<<dim3(static_cast<unsigned>((waves + RF_WAVES - 1) / RF_WAVES)), dim3(RF_WAVES * 64), 0,
                            p.stream>>>(q, k, v, p.out, ra.list, ra.guard, n, 1.0 / p.h, p.lambda);
        prof_end(p.stream);
    }
    return hipGetLastError();
}

}  // namespace lla
