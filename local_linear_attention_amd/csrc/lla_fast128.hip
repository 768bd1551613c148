// Matrix-core path of the causal LLA forward for bf16 inputs, head dimension 128.
//
// The estimator and its centred form are those of the "Parallax" blog post, section 2
// "Canonical Formulation" (local linear fit with softmax-kernel weights and a ridge) and
// Appendix E (rank-one split of the moment matrix); the per-row shift is the safe-softmax
// maximum of the arXiv page's scoring-form paragraph, applied to the weights and the ridge.
// Per query row i of a head, with wt_ij = e^{q_i.k_j/h - m_i}:
//   b_i = vbar_i - C_vk (C_kk + lambda e^{-m_i} I)^{-1} (kbar_i - q_i).
// The cross moment C_vk is never formed: it reaches y_i = (C_kk + ...)^{-1}(kbar_i - q_i)
// through a second, attention-like sweep over the prefix (the probe pass),
//   b_i = a_v + (1/omega') sum_j w_ij t_ij (v_j - a_v),
//   t_ij = 1 + S_k.yh_i / omega' - (k_j - a).yh_i,   yh_i = omega' y_i,
// which equals vbar_i - C_vk y_i because the weighted sum of k_j - kbar_i vanishes.
//
// Work split (rows are query positions i of one head, d = 128):
//   * rows i < 4d run on the fp64 kernel (prefixes of at most 4d keys: C_kk is rank-deficient
//     or poorly conditioned there; in fp16 the rows just past 2d reach about 2e-3, and with
//     keys 64 times larger than the queries rows [2d, 4d) pass the 3e-3 bar unseen by the
//     check below);
//   * rows i >= 4d:
//       lla8_anchor_kernel  per-head sums of the keys and values of positions [0, 2d): the
//                           centring anchor a (every row here has them in its prefix);
//       lla8_pack_kernel    per 64-key tile: K and V feature-major as fp16(x - a) (one
//                           rounding), K key-major as given (bf16) and centred (fp16);
//       lla8_rowmax_kernel  score pass on MFMA (bf16) with a running max: m_i;
//       lla8_keymom_kernel  per query, sw = fp16(e^{(s - m)/2}), R = fp16(sw (k - a)),
//                           C = R^T R on MFMA (36 upper 16x16 blocks, fp32 accumulate), block
//                           sums S_k = sum w (k - a), omega' = sum w with w = fp16(sw^2); the
//                           rank-one downdate and ridge, a blocked LDL^T solve in one wave;
//       lla8_probe_kernel   the probe pass on MFMA, bitwise the same scores and weights, and
//                           the per-row reproduction check;
//       lla_exact_list_kernel  the rows handed back, in fp64.
//
// MFMA v_mfma_f32_16x16x32_{bf16,f16}: lane l supplies row/column (l % 16) of A/B and K-slots
// 8 (l / 16) .. +8; D[4 (l / 16) + r][l % 16] is accumulator register r of lane l.
#include "lla_device.h"
#include "lla_internal.h"

#include <math.h>

#include <mutex>
#include <type_traits>

namespace lla {
namespace {

constexpr int D8 = 128;                      // head dimension of this path
constexpr int T8 = 64;                       // keys per tile
constexpr int NW8 = 4;                       // waves per block
constexpr int F_LD = T8 + 8;                 // feature-major fp16 row: 64 keys + 8 halves padding (144 B)
constexpr int F_BYTES = D8 * F_LD * 2;       // one tile of K (or V) feature-major: 18 KiB
constexpr int K_LD = D8 + 8;                 // key-major row: 128 features + 8 halves padding (272 B)
constexpr int KM_BYTES = T8 * K_LD * 2;      // one tile key-major: 17 KiB
constexpr int KM_STRIDE8 = 2 * KM_BYTES;     // workspace: bf16 keys as given, then fp16 centred keys
// Check image of a tile: projections of the centred keys on the Walsh functions of index
// 4t + 1 (fp16, [direction][key] rows of F_LD halves), then |v - a_v|^2 per key (fp32).
constexpr int KU8_NRM = NCHK * F_LD * 2;
static_assert(KU8_NRM + T8 * 4 <= KU_TILE_BYTES, "check image layout");
__device__ __forceinline__ constexpr int chk8_mask(int t) { return 4 * t + 1; }
constexpr int A8_SLICES = 16;                // key slices of the anchor sums
static_assert(F_BYTES % 1024 == 0 && KM_BYTES % 1024 == 0, "tile images are whole wave copies");

// Upper 16x16 block (I, J), I <= J, of a symmetric 128x128 matrix held as 36 accumulators.
__device__ __forceinline__ constexpr int ub8(int I, int J) { return I * 8 - I * (I - 1) / 2 + (J - I); }

// ---------------------------------------------------------------------------------------
// Anchor, pass 1: block (head, slice) sums its slice of positions [0, min(n, 2d)) of K and V
// per feature (fp32).  Thread -> 8 features (16 B) of K (groups 0-15) or V (16-31), every 8th
// key of the slice; the 8 key phases are added up through LDS.
__global__ __launch_bounds__(256) void lla8_anchor_kernel(const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v,
                                                          float* __restrict__ partial,
                                                          unsigned* __restrict__ guard, int n) {
    constexpr int NG = 2 * D8 / 8, NPH = 256 / NG;
    __shared__ float sums[NPH][2 * D8 + 4];
    const int bh = static_cast<int>(blockIdx.x) / A8_SLICES;
    const int sl = static_cast<int>(blockIdx.x) % A8_SLICES;
    const int tid = threadIdx.x, fgrp = tid % NG, ph = tid / NG;
    if (sl == 0 && tid < 2) guard[1 + 2 * bh + tid] = 0u;   // the head's range maxima
    if (blockIdx.x == 0 && tid == 2) guard[0] = 0u;         // no rows handed back yet
    const int na = min(n, 2 * D8);
    const int len = (na + A8_SLICES - 1) / A8_SLICES;
    const int j_lo = sl * len, j_hi = min(na, j_lo + len);
    const uint16_t* src = (fgrp < NG / 2 ? k : v) + static_cast<int64_t>(bh) * n * D8 + 8 * (fgrp % (NG / 2));
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = j_lo + ph; j < j_hi; j += NPH) {
        const uint4 x = *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(j) * D8);
        const uint32_t wds[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[e] += __uint_as_float((e & 1) ? (wds[e >> 1] & 0xffff0000u) : (wds[e >> 1] << 16));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) sums[ph][8 * fgrp + e] = acc[e];
    __syncthreads();
    {
        float tot = 0.0f;
#pragma unroll
        for (int p2 = 0; p2 < NPH; ++p2) tot += sums[p2][tid];
        partial[(static_cast<int64_t>(bh) * A8_SLICES + sl) * 2 * D8 + tid] = tot;
    }
}

__device__ __forceinline__ float bf16_elem(const uint4& x, int e) {
    const uint32_t w = e < 2 ? x.x : e < 4 ? x.y : e < 6 ? x.z : x.w;
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
}

// Pack one 64-key tile (keys past n are zero): K and V feature-major as fp16(x - a) (rows of
// F_LD halves), K key-major as given (bf16) and as the same fp16(k - a) values (rows of K_LD
// halves), all padding zero; tile 0 of a head also writes the head's anchor.  The anchor
// a = fp16(mean over positions [0, min(n, 2d))) of the keys and of the values.
// Thread -> key pair (2 pr, 2 pr + 1) and feature groups fg, fg + 8 (8 features each).
__global__ __launch_bounds__(256) void lla8_pack_kernel(const uint16_t* __restrict__ k,
                                                        const uint16_t* __restrict__ v,
                                                        const float* __restrict__ partial,
                                                        float* __restrict__ anchors,
                                                        unsigned char* __restrict__ kf,
                                                        unsigned char* __restrict__ vf,
                                                        unsigned char* __restrict__ km,
                                                        unsigned char* __restrict__ kuf,
                                                        unsigned* __restrict__ guard, int n, int ntiles) {
    __shared__ float anc[2 * D8];
    __shared__ float ys[T8][16][3];     // per key and feature group: the 8-point transforms kept
    __shared__ float vpart[8][T8];      // |v - a_v|^2 over each thread's 16 features
    __shared__ float wmax[4][2];        // per wave: largest |k - a|, |v - a_v|
    const int bh = static_cast<int>(blockIdx.x) / ntiles, t = static_cast<int>(blockIdx.x) % ntiles;
    const int tid = threadIdx.x;
    {
        float sum = 0.0f;
        for (int sl = 0; sl < A8_SLICES; ++sl)
            sum += partial[(static_cast<int64_t>(bh) * A8_SLICES + sl) * 2 * D8 + tid];
        anc[tid] = static_cast<float>(static_cast<_Float16>(sum / static_cast<float>(min(n, 2 * D8))));
        if (t == 0) anchors[static_cast<int64_t>(bh) * 2 * D8 + tid] = anc[tid];
    }
    __syncthreads();
    const int pr = tid & 31;
    const int64_t base = static_cast<int64_t>(bh) * n * D8;
    const int ja = t * T8 + 2 * pr, jb = ja + 1;
    const int64_t tile = static_cast<int64_t>(bh) * ntiles + t;
    unsigned char* kmt = km + tile * KM_STRIDE8;
    uint32_t* kft = reinterpret_cast<uint32_t*>(kf + tile * F_BYTES);
    uint32_t* vft = reinterpret_cast<uint32_t*>(vf + tile * F_BYTES);
    float mk = 0.0f, mv = 0.0f;   // the largest centred magnitudes, for the range guard
    float vsa = 0.0f, vsb = 0.0f;  // |v - a_v|^2 of keys 2p, 2p+1 over this thread's features
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int fg = (tid >> 5) + 8 * it;   // features 8 fg .. 8 fg + 7
        uint4 k0 = make_uint4(0, 0, 0, 0), k1 = k0, v0 = k0, v1 = k0;
        if (ja < n) {
            k0 = *reinterpret_cast<const uint4*>(k + base + static_cast<int64_t>(ja) * D8 + 8 * fg);
            v0 = *reinterpret_cast<const uint4*>(v + base + static_cast<int64_t>(ja) * D8 + 8 * fg);
        }
        if (jb < n) {
            k1 = *reinterpret_cast<const uint4*>(k + base + static_cast<int64_t>(jb) * D8 + 8 * fg);
            v1 = *reinterpret_cast<const uint4*>(v + base + static_cast<int64_t>(jb) * D8 + 8 * fg);
        }
        half8 ca, cb, va, vb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float ak = anc[8 * fg + e], av = anc[D8 + 8 * fg + e];
            ca[e] = static_cast<_Float16>(ja < n ? bf16_elem(k0, e) - ak : 0.0f);
            cb[e] = static_cast<_Float16>(jb < n ? bf16_elem(k1, e) - ak : 0.0f);
            va[e] = static_cast<_Float16>(ja < n ? bf16_elem(v0, e) - av : 0.0f);
            vb[e] = static_cast<_Float16>(jb < n ? bf16_elem(v1, e) - av : 0.0f);
            if (ja < n) {
                mk = fmaxf(mk, fabsf(bf16_elem(k0, e) - ak));
                mv = fmaxf(mv, fabsf(bf16_elem(v0, e) - av));
            }
            if (jb < n) {
                mk = fmaxf(mk, fabsf(bf16_elem(k1, e) - ak));
                mv = fmaxf(mv, fabsf(bf16_elem(v1, e) - av));
            }
        }
        // key-major: bf16 as given, then centred fp16; padding (bytes 256..271 of a row) zero
        *reinterpret_cast<uint4*>(kmt + (2 * pr) * (K_LD * 2) + 16 * fg) = k0;
        *reinterpret_cast<uint4*>(kmt + (2 * pr + 1) * (K_LD * 2) + 16 * fg) = k1;
        *reinterpret_cast<half8*>(kmt + KM_BYTES + (2 * pr) * (K_LD * 2) + 16 * fg) = ca;
        *reinterpret_cast<half8*>(kmt + KM_BYTES + (2 * pr + 1) * (K_LD * 2) + 16 * fg) = cb;
        if (fg == 15) {
            const uint4 z = make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4*>(kmt + (2 * pr) * (K_LD * 2) + 2 * D8) = z;
            *reinterpret_cast<uint4*>(kmt + (2 * pr + 1) * (K_LD * 2) + 2 * D8) = z;
            *reinterpret_cast<uint4*>(kmt + KM_BYTES + (2 * pr) * (K_LD * 2) + 2 * D8) = z;
            *reinterpret_cast<uint4*>(kmt + KM_BYTES + (2 * pr + 1) * (K_LD * 2) + 2 * D8) = z;
        }
        // feature-major: row f holds keys (2 pr, 2 pr + 1) in its 32-bit word pr
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int f = 8 * fg + e;
            vsa = fmaf(static_cast<float>(va[e]), static_cast<float>(va[e]), vsa);
            vsb = fmaf(static_cast<float>(vb[e]), static_cast<float>(vb[e]), vsb);
            const h16x2 kk = {ca[e], cb[e]}, vv = {va[e], vb[e]};
            kft[f * (F_LD / 2) + pr] = __builtin_bit_cast(uint32_t, kk);
            vft[f * (F_LD / 2) + vcol(2 * pr) / 2] = __builtin_bit_cast(uint32_t, vv);
            if (pr < (F_LD - T8) / 2) {
                kft[f * (F_LD / 2) + T8 / 2 + pr] = 0u;
                vft[f * (F_LD / 2) + T8 / 2 + pr] = 0u;
            }
        }
        // check image, first stage: 8-point transforms over this feature group (ml = 1, 5)
        float xa[8], xb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            xa[e] = static_cast<float>(ca[e]);
            xb[e] = static_cast<float>(cb[e]);
        }
        walsh_transform(xa);
        walsh_transform(xb);
        ys[2 * pr][fg][0] = xa[1];
        ys[2 * pr][fg][1] = xa[5];
        ys[2 * pr + 1][fg][0] = xb[1];
        ys[2 * pr + 1][fg][1] = xb[5];
    }
    mk = wave_max_nonneg(mk);
    mv = wave_max_nonneg(mv);
    if ((tid & 63) == 0) {
        wmax[tid >> 6][0] = mk;
        wmax[tid >> 6][1] = mv;
    }
    vpart[tid >> 5][2 * pr] = vsa;
    vpart[tid >> 5][2 * pr + 1] = vsb;
    __syncthreads();
    if (tid == 0) {   // the block's range maxima, one atomic each
        float bk = 0.0f, bv = 0.0f;
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
            bk = fmaxf(bk, wmax[w4][0]);
            bv = fmaxf(bv, wmax[w4][1]);
        }
        atomicMax(guard + 1 + 2 * bh, __float_as_uint(bk));
        atomicMax(guard + 2 + 2 * bh, __float_as_uint(bv));
    }
    // Check image: the 128-point Walsh-Hadamard transform of each key's centred values,
    // X[m] = sum_f (-1)^popcount(f & m) x_f with f = 8 fh + e and m = 8 mh + ml, splits into
    // 8-point transforms over e (in the loop above, per thread and feature group; ml of 1 and
    // 5 kept) and 16-point transforms over fh (here, per key); the directions are
    // m = 4t + 1, i.e. t = 2 mh + (ml == 5).
    unsigned char* kut = kuf + tile * KU_TILE_BYTES;
    {   // thread -> key j, ml = 1 + 4 s, half hb of the mh range
        const int j = tid & (T8 - 1), sl = (tid >> 6) & 1, hb = tid >> 7;
        float x16[16];
#pragma unroll
        for (int g16 = 0; g16 < 16; ++g16) x16[g16] = ys[j][g16][sl];
        walsh_transform(x16);
        _Float16* kur = reinterpret_cast<_Float16*>(kut);
#pragma unroll
        for (int u8 = 0; u8 < 8; ++u8) {
            const int mh = 8 * hb + u8;
            kur[(2 * mh + sl) * F_LD + vcol(j)] = static_cast<_Float16>(hb ? x16[8 + u8] : x16[u8]);
        }
        if (tid < T8) {
            float nv = 0.0f;
#pragma unroll
            for (int f8 = 0; f8 < 8; ++f8) nv += vpart[f8][j];
            reinterpret_cast<float*>(kut + KU8_NRM)[j] = nv;
        }
    }
    if (tid < NCHK) {   // row padding of the projections
        *reinterpret_cast<uint4*>(kut + tid * F_LD * 2 + T8 * 2) = make_uint4(0, 0, 0, 0);
    } else if (tid < NCHK + 16) {   // tail after the norms
        *reinterpret_cast<uint4*>(kut + KU8_NRM + T8 * 4 + (tid - NCHK) * 16) = make_uint4(0, 0, 0, 0);
    }
}

// ---------------------------------------------------------------------------------------
// Score pass with a running max (rows i >= row0): m_i = max_{j <= i} q_i.k_j / h in log2
// units.  Block = 4 waves x 2 sets of 16 queries (the sets share the key operands); 64-key
// tiles of the bf16 key-major image stream through a ring of three LDS buffers, copied
// straight from the workspace; S^T block kb of a tile on MFMA (four 32-feature steps):
// lane (g, c) register r = key 16 kb + 4 g + r, query c of the set.
constexpr int R8_SETS = 2, R8_QW = 16 * R8_SETS, R8_QB = NW8 * R8_QW;
constexpr int R8_LOADS = KM_BYTES / 1024;                    // 17 wave copies per tile
constexpr int R8_WLOADS = (R8_LOADS + NW8 - 1) / NW8;        // 5 per wave (surplus repeats the last)

__global__ __launch_bounds__(256) void lla8_rowmax_kernel(const uint16_t* __restrict__ q,
                                                          const unsigned char* __restrict__ km,
                                                          float* __restrict__ mrow, int n, int row0, int BH,
                                                          float sl2) {
    __shared__ __attribute__((aligned(16))) unsigned char ring[3 * KM_BYTES];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int g = lane >> 4, c = lane & 15;
    const int nrows = n - row0;
    const int nblk = (nrows + R8_QB - 1) / R8_QB;
    int blk, bh;
    head_major_block(static_cast<int>(blockIdx.x), BH, nblk, &bh, &blk);
    const int q0 = row0 + blk * R8_QB;
    const int qlast = min(q0 + R8_QB, n) - 1;
    const int wave_first = q0 + wu * R8_QW;
    const int wave_last = min(wave_first + R8_QW - 1, n - 1);
    const int64_t base = static_cast<int64_t>(bh) * n * D8;
    int qi[R8_SETS], qc[R8_SETS];
    bf16x8 qf[R8_SETS][4];
#pragma unroll
    for (int st = 0; st < R8_SETS; ++st) {
        qi[st] = wave_first + 16 * st + c;
        qc[st] = min(qi[st], n - 1);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qf[st][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(
                                                        q + base + static_cast<int64_t>(qc[st]) * D8 + ks * 32 + 8 * g));
    }
    const int ntiles = qlast / T8 + 1;
    const int ptiles = (n + T8 - 1) / T8;
    const __amdgpu_buffer_rsrc_t img = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(uniform_ptr(km + static_cast<int64_t>(bh) * ptiles * KM_STRIDE8)), 0,
        ptiles * KM_STRIDE8, 0x00020000);
    int voff[R8_WLOADS];
#pragma unroll
    for (int e = 0; e < R8_WLOADS; ++e) voff[e] = lane * 16 + min(wu + NW8 * e, R8_LOADS - 1) * 1024;
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ring));
    auto issue = [&](int tt) {
        const int ts = min(tt, ntiles - 1);
        const uint32_t dst = lds0 + static_cast<uint32_t>((tt % 3) * KM_BYTES);
#pragma unroll
        for (int e = 0; e < R8_WLOADS; ++e) {
            const int u = min(wu + NW8 * e, R8_LOADS - 1);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                img, reinterpret_cast<__attribute__((address_space(3))) void*>(static_cast<uintptr_t>(dst + u * 1024)),
                16, voff[e], ts * KM_STRIDE8, 0, 0);
        }
    };
    // Only tile copies are in flight in the loop: after tile t+1's come tile t+2's
    // R8_WLOADS, so vmcnt <= R8_WLOADS means tile t+1 has landed.
    auto next_tile = [] {
        __builtin_amdgcn_s_waitcnt(R8_WLOADS | (0x7 << 4) | (0xF << 8));
        LDS_FENCE();
        __builtin_amdgcn_s_barrier();
        LDS_FENCE();
    };
    float m_run[R8_SETS];
#pragma unroll
    for (int st = 0; st < R8_SETS; ++st) m_run[st] = -INFINITY;
    issue(0);
    issue(1);
    next_tile();
    for (int t = 0; t < ntiles; ++t) {
        issue(t + 2);
        const int j0 = t * T8;
        auto tile_body = [&](auto masked) {
            const unsigned char* cur = ring + (t % 3) * KM_BYTES;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                bf16x8 a[4];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    a[ks] = __builtin_bit_cast(
                        bf16x8, *reinterpret_cast<const uint4*>(cur + (kb * 16 + c) * (K_LD * 2) + ks * 64 + 16 * g));
#pragma unroll
                for (int st = 0; st < R8_SETS; ++st) {
                    float4v s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) s = mfma_bf16(a[ks], qf[st][ks], s);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = j0 + kb * 16 + 4 * g + r;
                        m_run[st] = fmaxf(m_run[st], (!decltype(masked)::value || j <= qc[st]) ? s[r] : -INFINITY);
                    }
                }
            }
        };
        if (j0 + T8 - 1 <= wave_first) tile_body(std::false_type{});
        else if (j0 <= wave_last) tile_body(std::true_type{});   // wave-uniform
        next_tile();
    }
    __builtin_amdgcn_s_waitcnt(0x0 | (0x7 << 4) | (0xF << 8));   // copies past the last tile
#pragma unroll
    for (int st = 0; st < R8_SETS; ++st) {
        float m = fmaxf(m_run[st], __shfl_xor(m_run[st], 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        if (g == 0 && qi[st] < n) mrow[static_cast<int64_t>(bh) * nrows + (qi[st] - row0)] = m * sl2;
    }
}

// ---------------------------------------------------------------------------------------
// Key moments and solve (rows i >= row0).  Block = 8 waves, one query each (8 consecutive
// rows), two waves per SIMD: a wave's 36 accumulator blocks (144 registers) plus its
// operands fit the 256 registers a wave has at that occupancy, and the 8 queries share
// every tile the block brings into LDS.
// Two LDS rings advance together: the fp16 centred key image (feature-major, with each
// tile's weights) and the bf16 key image (key-major, the score operand), the latter one
// tile ahead.  Step t copies key image t + 2 and score image t + 3 straight from the
// workspace; waves 0-3 take the scores of 16 keys each of tile t + 1 for the 8 queries (four
// bf16 MFMAs) and store sqrt-weights sw and fp16 weights w = fp16(sw^2) per query; per
// 32-key half of tile t, every wave reads the key image, forms R = sw (k - a) for its query
// (packed fp16 multiplies) and accumulates the 36 upper blocks of C = R^T R, plus the block
// sums S_k of the 8 queries for feature block w.  Keys past a query carry weight zero: one
// straight-line block per half, no per-query branches.
constexpr int KW8 = 8;                                // waves per block
constexpr int K8_BQ = KW8;                            // queries per block, one per wave
constexpr int K8_SW = F_BYTES;                        // sqrt-weights [query][key], rows of F_LD halves
constexpr int K8_SW2 = K8_SW + K8_BQ * F_LD * 2;      // fp16 weights, 16 rows (rows >= 8 zero)
constexpr int K8_BUF = K8_SW2 + 16 * F_LD * 2;        // key-image ring buffer
constexpr int K8_LOADS = F_BYTES / 1024;              // 18 wave copies per key image
constexpr int K8_WLOADS = (K8_LOADS + KW8 - 1) / KW8; // 3 per wave (surplus repeats the last)
constexpr int K8_SLOADS = KM_BYTES / 1024;            // 17 wave copies per score image
constexpr int K8_WSLOADS = (K8_SLOADS + KW8 - 1) / KW8;
constexpr int K8_NBUF = 3;
constexpr int K8_SRING = K8_NBUF * K8_BUF;            // score-image ring after the key-image ring
constexpr int K8_RING = K8_SRING + K8_NBUF * KM_BYTES;
constexpr int S8_LD = D8 + 4;                         // solve staging row stride (floats)
constexpr int S8_FLOATS = 16 * S8_LD + 16;            // per wave: a block row of 16 + 16 pivots
constexpr int K8_SOLVE_BYTES = KW8 * S8_FLOATS * 4;
constexpr int K8_MEAN_OFF = K8_RING > K8_SOLVE_BYTES ? K8_RING : K8_SOLVE_BYTES;
constexpr int K8_SMEM = K8_MEAN_OFF + (K8_BQ * D8 + 4 * 16) * 4;
static_assert(K8_SMEM <= 160 * 1024, "one block per CU");
constexpr int P8_YLD = 2 * D8;                        // per query: yh hi (fp16) | yh lo (fp16)
constexpr int P8_QSC = 8;                             // per query: gamma, 2^-e, 1/omega', dropped-pivot flag,
                                                      // weighted mean |k - a|^2, 3 unused
constexpr int P8_CHK = NCHK;                          // per query: the check's target (below)
static_assert(K8_BUF % 16 == 0 && K8_SRING % 16 == 0 && K8_MEAN_OFF % 16 == 0, "LDS areas stay 16-byte aligned");
static_assert(K8_BQ <= 16, "score MFMA has 16 query columns");

// Sums and maxima over the 64 lanes of a wave (every lane gets the result): DPP within each
// row of 16 lanes, then the four row results by readlane.
template <int CTRL>
__device__ __forceinline__ float dpp8(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float wave_sum8(float x) {
    x += dpp8<0xB1>(x);    // quad_perm [1, 0, 3, 2]
    x += dpp8<0x4E>(x);    // quad_perm [2, 3, 0, 1]
    x += dpp8<0x141>(x);   // row_half_mirror
    x += dpp8<0x140>(x);   // row_mirror
    return (lane_value(x, 0) + lane_value(x, 16)) + (lane_value(x, 32) + lane_value(x, 48));
}
__device__ __forceinline__ float row_sum8(float x) {   // over each row of 16 lanes
    x += dpp8<0xB1>(x);
    x += dpp8<0x4E>(x);
    x += dpp8<0x141>(x);
    return x + dpp8<0x140>(x);
}
__device__ __forceinline__ float wave_max8(float x) {
    x = fmaxf(x, dpp8<0xB1>(x));
    x = fmaxf(x, dpp8<0x4E>(x));
    x = fmaxf(x, dpp8<0x141>(x));
    x = fmaxf(x, dpp8<0x140>(x));
    return fmaxf(fmaxf(lane_value(x, 0), lane_value(x, 16)), fmaxf(lane_value(x, 32), lane_value(x, 48)));
}

// Panel K of one query's solve (A y = z, A = C - s s^T iom + lam I, 128 x 128 SPD,
// iom = 1 / omega') in one wave, a blocked LDL^T factorisation in place:
//   ckk: the 36 upper blocks of C in accumulator layout (lane (g, c) register r of block
//        (I, J) = C[16 I + 4 g + r][16 J + c]).  The trailing blocks (I, J > K) take the update
//        C_IJ -= L_IK D_K L_JK^T on 16x16x4 fp32 MFMAs; block row K is replaced by the
//        multipliers, L[16 J + c][16 K + 4 g + r] in register r of block (K, J).
//   z[h]: right-hand side of row lane + 64 h, forward-eliminated as the pivots pass.
//   dd[K]: pivot d of row 16 K + c (lane (g, c)).
//   skq: s in LDS; Sg: this wave's LDS staging area.
// Block row K is staged through LDS with the rank-one downdate and the ridge applied to
// each entry once (the trailing updates are linear, so the downdate commutes with them) and
// read back lane-per-row (lane holds rows lane and lane + 64); pivots are broadcast with
// readlane; the multipliers go back through LDS, to the trailing update's operands and to
// their place.
template <int K>
__device__ __forceinline__ void panel8(float4v (&ckk)[36], float (&z)[2], float (&dd)[8], const float thr,
                                       const float lam, const float iom, const float* skq, float* Sg,
                                       const int lane, const int g, const int c) {
    constexpr int H0 = K < 4 ? 0 : 1;   // rows lane < 64 lie above every panel K >= 4
    constexpr int HP = (16 * K) / 64;   // the pivot rows of this panel are rows lane + 64 HP
    float* Dg = Sg + 16 * S8_LD;
    {
        float srow[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) srow[r] = skq[16 * K + 4 * g + r] * iom;
#pragma unroll
        for (int J = K; J < 8; ++J) {
            const float scol = skq[16 * J + c];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float val = fmaf(-srow[r], scol, ckk[ub8(K, J)][r]);
                if (J == K && 4 * g + r == c) val += lam;
                Sg[(4 * g + r) * S8_LD + 16 * J + c] = val;
            }
        }
    }
    LDS_FENCE();
    float Lf[2][16];
#pragma unroll
    for (int h = H0; h < 2; ++h)
#pragma unroll
        for (int t = 0; t < 16; ++t) Lf[h][t] = Sg[t * S8_LD + lane + 64 * h];
    LDS_FENCE();
    // Rows above the panel (lanes < 16 K when HP = 0) read stale words; their multipliers
    // are zero (row test), so those never reach a live value.
#pragma unroll
    for (int p = 0; p < 16; ++p) {
        const int P = 16 * K + p, lp = P - 64 * HP;
        const float piv = lane_value(Lf[HP][p], lp);
        // Reciprocal pivot (about 1 ulp); a dropped pivot gets a zero column of L.
        const float inv = piv > thr ? __builtin_amdgcn_rcpf(piv) : 0.0f;
        int row = lane;
        asm volatile("" : "+v"(row));   // row tests per step: no precomputed lane masks
        float f[2];
#pragma unroll
        for (int h = H0; h < 2; ++h) {
            if (h > HP) f[h] = Lf[h][p] * inv;   // rows lane + 64 > P for every P < 64
            else f[h] = row > lp ? Lf[h][p] * inv : 0.0f;
        }
        const float zp = lane_value(z[HP], lp);
#pragma unroll
        for (int h = H0; h < 2; ++h) z[h] = fmaf(-f[h], zp, z[h]);
#pragma unroll
        for (int t = p + 1; t < 16; ++t) {
            const float bt = lane_value(Lf[HP][t], lp);
#pragma unroll
            for (int h = H0; h < 2; ++h) Lf[h][t] = fmaf(-f[h], bt, Lf[h][t]);
        }
        int col = c;
        asm volatile("" : "+v"(col));
        dd[K] = col == p ? piv : dd[K];
#pragma unroll
        for (int h = H0; h < 2; ++h) Lf[h][p] = f[h];
    }
    // Multipliers Sg[t][a] = L[a][16 K + t]; the panel's pivots Dg[t] = d[16 K + t].
#pragma unroll
    for (int h = H0; h < 2; ++h)
#pragma unroll
        for (int t = 0; t < 16; ++t) Sg[t * S8_LD + lane + 64 * h] = Lf[h][t];
    if (g == 0) Dg[c] = dd[K];
    LDS_FENCE();
#pragma unroll
    for (int J = K; J < 8; ++J)
#pragma unroll
        for (int r = 0; r < 4; ++r) ckk[ub8(K, J)][r] = Sg[(4 * g + r) * S8_LD + 16 * J + c];
    if constexpr (K < 7) {
        // Trailing update over the panel columns 16 K + 4 s + g (K-slot g of step s); the
        // operands of block row I are read when its blocks are updated.
        float dv[4];
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) dv[s4] = Dg[4 * s4 + g];
#pragma unroll
        for (int I = K + 1; I < 8; ++I) {
            float LoI[4];
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) LoI[s4] = -Sg[(4 * s4 + g) * S8_LD + 16 * I + c];
#pragma unroll
            for (int J = I; J < 8; ++J)
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4)
                    ckk[ub8(I, J)] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                        LoI[s4], dv[s4] * Sg[(4 * s4 + g) * S8_LD + 16 * J + c], ckk[ub8(I, J)], 0, 0, 0);
        }
    }
    LDS_FENCE();
}

// One query's solve.  Returns y[J] = y[16 J + c] in lane (g, c) (the same in every g).
__device__ __forceinline__ void solve8(float4v (&ckk)[36], float (&z)[2], const float thr, const float lam,
                                       const float iom, const float* skq, float* Sg, float (&y)[8],
                                       float& dropped, const int lane, const int g, const int c) {
    float dd[8];
#pragma unroll
    for (int J = 0; J < 8; ++J) dd[J] = 0.0f;
    panel8<0>(ckk, z, dd, thr, lam, iom, skq, Sg, lane, g, c);
    __builtin_amdgcn_sched_barrier(0);
    panel8<1>(ckk, z, dd, thr, lam, iom, skq, Sg, lane, g, c);
    __builtin_amdgcn_sched_barrier(0);
    panel8<2>(ckk, z, dd, thr, lam, iom, skq, Sg, lane, g, c);
    __builtin_amdgcn_sched_barrier(0);
    panel8<3>(ckk, z, dd, thr, lam, iom, skq, Sg, lane, g, c);
    __builtin_amdgcn_sched_barrier(0);
    panel8<4>(ckk, z, dd, thr, lam, iom, skq, Sg, lane, g, c);
    __builtin_amdgcn_sched_barrier(0);
    panel8<5>(ckk, z, dd, thr, lam, iom, skq, Sg, lane, g, c);
    __builtin_amdgcn_sched_barrier(0);
    panel8<6>(ckk, z, dd, thr, lam, iom, skq, Sg, lane, g, c);
    __builtin_amdgcn_sched_barrier(0);
    panel8<7>(ckk, z, dd, thr, lam, iom, skq, Sg, lane, g, c);
    __builtin_amdgcn_sched_barrier(0);
    // x = D^{-1} z (zero at dropped pivots) in the distributed layout: x[J] = x[16 J + c].
#pragma unroll
    for (int h = 0; h < 2; ++h) Sg[lane + 64 * h] = z[h];
    LDS_FENCE();
    float x[8];
    float drop = 0.0f;   // 1 if a pivot of this lane's rows was dropped
#pragma unroll
    for (int J = 0; J < 8; ++J) {
        float inv_d = __builtin_amdgcn_rcpf(dd[J]);
        inv_d = fmaf(inv_d, fmaf(-dd[J], inv_d, 1.0f), inv_d);   // one Newton step: ~0.5 ulp
        x[J] = dd[J] > thr ? Sg[16 * J + c] * inv_d : 0.0f;
        drop = dd[J] > thr ? drop : 1.0f;
        y[J] = 0.0f;
    }
    dropped = wave_max8(drop);
    LDS_FENCE();
    // Back substitution L^T y = x from the last row: y_P = x_P - sum_{b > P} L[b][P] y_b.
    // For P = 16 K + 4 g' + r', L[16 J + c][P] is register r' of block (K, J) in lane (g', c):
    // the products of row g' of lanes are summed over its 16 lanes (L[b][P] is zero for
    // b <= P, and y of rows not yet solved is zero), and the sum goes to every lane.
#pragma unroll
    for (int K = 7; K >= 0; --K)
#pragma unroll
        for (int p = 15; p >= 0; --p) {
            float part = 0.0f;
#pragma unroll
            for (int J = K; J < 8; ++J) part = fmaf(ckk[ub8(K, J)][p % 4], y[J], part);
            part += dpp8<0xB1>(part);
            part += dpp8<0x4E>(part);
            part += dpp8<0x141>(part);
            part += dpp8<0x140>(part);
            const float sum = lane_value(part, 16 * (p / 4));
            int col = c;
            asm volatile("" : "+v"(col));
            y[K] = col == p ? x[K] - sum : y[K];
        }
}

__global__ __launch_bounds__(KW8 * 64, 1) void lla8_keymom_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ mrow, const float* __restrict__ anchors,
    const unsigned char* __restrict__ kf, const unsigned char* __restrict__ km, _Float16* __restrict__ yhl,
    float* __restrict__ qsc, float* __restrict__ chk, const unsigned* __restrict__ guard, int n, int row0,
    int BH, float sl2, float lambda) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int g = lane >> 4, c = lane & 15;
    const int prows = n - row0;   // rows of this path, and of the row-max array
    const int nblk = (prows + K8_BQ - 1) / K8_BQ;
    int blk, bh;
    head_major_block(static_cast<int>(blockIdx.x), BH, nblk, &bh, &blk);
    const int i0 = row0 + blk * K8_BQ;
    const int last = min(i0 + K8_BQ - 1, n - 1);
    const int64_t base = static_cast<int64_t>(bh) * n * D8;
    if (head_unsafe(guard, bh)) return;   // block-uniform: the probe pass hands the rows back

    // Rows K8_BQ.. of every weight buffer: the zero rows of the block-sum MFMA operand.
    for (int e = tid; e < K8_NBUF * (16 - K8_BQ) * F_LD / 8; e += KW8 * 64) {
        const int bsel = e / ((16 - K8_BQ) * F_LD / 8), rem = e % ((16 - K8_BQ) * F_LD / 8);
        *reinterpret_cast<uint4*>(smem + bsel * K8_BUF + K8_SW2 + K8_BQ * F_LD * 2 + rem * 16) = make_uint4(0, 0, 0, 0);
    }
    // Score operand (waves 0-3): column c < 8 is query i0 + c (the other columns are zero).
    const bool scorer = wu < 4;
    const int qcol = min(i0 + c, n - 1);
    const bool colv = c < K8_BQ;
    const float mcol = mrow[static_cast<int64_t>(bh) * prows + (qcol - row0)];   // log2 units
    bf16x8 qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (colv) raw = *reinterpret_cast<const uint4*>(q + base + static_cast<int64_t>(qcol) * D8 + ks * 32 + 8 * g);
        qf[ks] = __builtin_bit_cast(bf16x8, raw);
    }
    float om2p = 0.0f;   // fp16 weights of query c summed over this lane's keys
    const float hs = 0.5f * sl2, hm = 0.5f * mcol;
    auto kbuf = [&](int tt) { return smem + (tt % K8_NBUF) * K8_BUF; };
    auto sbuf = [&](int tt) { return smem + K8_SRING + (tt % K8_NBUF) * KM_BYTES; };
    // Scores of key block w (16 keys) of tile tt from its score image: lane (g, c) register
    // r = key 16 w + 4 g + r, query c; sqrt-weights and fp16 weights into the key buffer of tt.
    // The MFMAs are issued before the tile's key moments and their results used after the
    // first half, so that the chain's latency hides behind the moment MFMAs.
    auto scores_mfma = [&](int tt) {
        const unsigned char* sb = sbuf(tt);
        float4v s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            s = mfma_bf16(*reinterpret_cast<const bf16x8*>(sb + (16 * wu + c) * (K_LD * 2) + 64 * ks + 16 * g), qf[ks], s);
        return s;
    };
    auto scores_store = [&](float4v s, int tt) {
        const int j0 = tt * T8;
        float e[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) e[rr] = __builtin_amdgcn_exp2f(fmaf(s[rr], hs, -hm));
        if (j0 + T8 - 1 > i0) {   // block-uniform: keys past some query of the block
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) e[rr] = j0 + 16 * wu + 4 * g + rr <= qcol ? e[rr] : 0.0f;
        }
        half4 sw4;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) sw4[rr] = static_cast<_Float16>(e[rr]);
        const half4 w4 = sw4 * sw4;
        if (colv) {
            unsigned char* kb = kbuf(tt);
            *reinterpret_cast<half4*>(reinterpret_cast<_Float16*>(kb + K8_SW) + c * F_LD + 16 * wu + 4 * g) = sw4;
            *reinterpret_cast<half4*>(reinterpret_cast<_Float16*>(kb + K8_SW2) + c * F_LD + 16 * wu + 4 * g) = w4;
            const h16x2 one = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
            om2p = __builtin_amdgcn_fdot2(__builtin_shufflevector(w4, w4, 0, 1), one, om2p, false);
            om2p = __builtin_amdgcn_fdot2(__builtin_shufflevector(w4, w4, 2, 3), one, om2p, false);
        }
    };

    float4v ckk[36];
#pragma unroll
    for (int b = 0; b < 36; ++b) ckk[b] = float4v{0.f, 0.f, 0.f, 0.f};
    // S_k of the block's queries: lane (g, c) register r = query 4 g + r, feature 16 w + c.
    float4v sk = {0.f, 0.f, 0.f, 0.f};

    const int ntiles = last / T8 + 1;
    const int ptiles = (n + T8 - 1) / T8;
    const __amdgpu_buffer_rsrc_t kimg = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(uniform_ptr(kf + static_cast<int64_t>(bh) * ptiles * F_BYTES)), 0,
        ptiles * F_BYTES, 0x00020000);
    const __amdgpu_buffer_rsrc_t simg = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(uniform_ptr(km + static_cast<int64_t>(bh) * ptiles * KM_STRIDE8)), 0,
        ptiles * KM_STRIDE8, 0x00020000);
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem));
    // Copies of key image tt into key buffer tt % 3 and of score image tt (the bf16 half of
    // the tile's key-major images) into score buffer tt % 3: wave w copies KiB chunks w,
    // w + 8, ...; every wave issues the same number of copies, surplus ones repeating the
    // last chunk.  Tiles past the last one re-read the last into buffers nobody reads again.
    auto issue_k = [&](int tt) {
        const int ts = min(tt, ntiles - 1);
        const uint32_t dst = lds0 + static_cast<uint32_t>((tt % K8_NBUF) * K8_BUF);
#pragma unroll
        for (int e = 0; e < K8_WLOADS; ++e) {
            const int u = min(wu + KW8 * e, K8_LOADS - 1);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                kimg, reinterpret_cast<__attribute__((address_space(3))) void*>(static_cast<uintptr_t>(dst + u * 1024)),
                16, lane * 16 + u * 1024, ts * F_BYTES, 0, 0);
        }
    };
    auto issue_s = [&](int tt) {
        const int ts = min(tt, ntiles - 1);
        const uint32_t dst = lds0 + static_cast<uint32_t>(K8_SRING + (tt % K8_NBUF) * KM_BYTES);
#pragma unroll
        for (int e = 0; e < K8_WSLOADS; ++e) {
            const int u = min(wu + KW8 * e, K8_SLOADS - 1);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                simg, reinterpret_cast<__attribute__((address_space(3))) void*>(static_cast<uintptr_t>(dst + u * 1024)),
                16, lane * 16 + u * 1024, ts * KM_STRIDE8, 0, 0);
        }
    };
    // Loads complete in order; after key image t + 1 and score image t + 2 come key image
    // t + 2 and score image t + 3, so vmcnt <= K8_WLOADS + K8_WSLOADS means the former two
    // have landed.  Encoding: vmcnt bits [3:0] and [15:14]; expcnt, lgkmcnt at their maxima.
    constexpr int K8_VM = K8_WLOADS + K8_WSLOADS;
    static_assert(K8_VM < 16, "vmcnt low bits");
    auto wait_tiles = [] {
        __builtin_amdgcn_s_waitcnt(K8_VM | (0x7 << 4) | (0xF << 8));
        LDS_FENCE();
    };
    // This wave's LDS stores are complete (lgkmcnt 0); loads still in flight (the images a
    // step ahead) are deliberately not waited for, which __syncthreads() would do.
    auto ring_barrier = [] {
        __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
        LDS_FENCE();
        __builtin_amdgcn_s_barrier();
        LDS_FENCE();
    };
    // Tile t, in two 32-key halves: R = sw (k - a) (one rounding, packed fp16 multiplies, in
    // place over the key rows), the 36 upper blocks of R^T R and the block sums of the 8
    // queries for feature block w.  The key rows of a half are read in two groups of four
    // feature blocks, each group's reads issued while the MFMAs of the previous group run:
    // group B of a half during the blocks within group A, group A of the next half during
    // the blocks within group B (the fences keep the reads from being hoisted further).
    auto compute_tile = [&](int t, bool second, auto&& after_first) {
        const unsigned char* cur = kbuf(t);
        const _Float16* Kt = reinterpret_cast<const _Float16*>(cur);
        const _Float16* Sw = reinterpret_cast<const _Float16*>(cur + K8_SW);
        const _Float16* Sw2 = reinterpret_cast<const _Float16*>(cur + K8_SW2);
        half8 ra[4], rb[4];
        auto read_group = [&](half8 (&r)[4], int fb0, int ko) {
#pragma unroll
            for (int fb = 0; fb < 4; ++fb) r[fb] = *reinterpret_cast<const half8*>(Kt + ((fb0 + fb) * 16 + c) * F_LD + ko);
        };
        read_group(ra, 0, 8 * g);
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            if (sub == 1 && !second) break;   // block-uniform: past every query of the block
            const int ko = 32 * sub + 8 * g;
            const half8 sw = *reinterpret_cast<const half8*>(Sw + wu * F_LD + ko);
            const half8 w8 = *reinterpret_cast<const half8*>(Sw2 + c * F_LD + ko);
            const half8 kw = *reinterpret_cast<const half8*>(Kt + (wu * 16 + c) * F_LD + ko);
#pragma unroll
            for (int fb = 0; fb < 4; ++fb) ra[fb] = ra[fb] * sw;
            LDS_FENCE();
            read_group(rb, 4, ko);
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int J = I; J < 4; ++J) ckk[ub8(I, J)] = mfma_f16(ra[I], ra[J], ckk[ub8(I, J)]);
            // The blocks within group A are issued before group B's rows are waited for.
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int J = I; J < 4; ++J) asm volatile("" : "+v"(ckk[ub8(I, J)]));
#pragma unroll
            for (int fb = 0; fb < 4; ++fb) asm volatile("" : "+v"(rb[fb]));
#pragma unroll
            for (int fb = 0; fb < 4; ++fb) rb[fb] = rb[fb] * sw;
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int J = 4; J < 8; ++J) ckk[ub8(I, J)] = mfma_f16(ra[I], rb[J - 4], ckk[ub8(I, J)]);
            sk = mfma_f16(w8, kw, sk);
            if (sub == 0) after_first();
            if (sub == 0 && second) {
                // the last uses of group A's rows are issued before the next half's rows land
                // in their registers
#pragma unroll
                for (int I = 0; I < 4; ++I)
#pragma unroll
                    for (int J = 4; J < 8; ++J) asm volatile("" : "+v"(ckk[ub8(I, J)]));
                LDS_FENCE();
                read_group(ra, 0, 32 + 8 * g);
            }
#pragma unroll
            for (int I = 4; I < 8; ++I)
#pragma unroll
                for (int J = I; J < 8; ++J) ckk[ub8(I, J)] = mfma_f16(rb[I - 4], rb[J - 4], ckk[ub8(I, J)]);
        }
    };
    // Prologue: score image 0, then (key image s + 2, score image s + 3) for s = -2, -1 as in
    // the loop.  Once score images 0 and 1 and key image 0 have landed, the scores of tile 0.
    issue_s(0);
    issue_k(0);
    issue_s(1);
    issue_k(1);
    issue_s(2);
    __builtin_amdgcn_s_waitcnt(K8_VM | (0x7 << 4) | (0xF << 8));   // s0, k0, s1 landed
    ring_barrier();
    if (scorer) scores_store(scores_mfma(0), 0);
    ring_barrier();
    // Step t: key image t and its weights are in LDS, and score image t + 1.
    for (int t = 0; t < ntiles; ++t) {
        issue_k(t + 2);
        issue_s(t + 3);
        float4v sv = {0.f, 0.f, 0.f, 0.f};
        if (scorer) sv = scores_mfma(t + 1);
        compute_tile(t, t * T8 + 32 <= last, [&] {
            if (scorer) scores_store(sv, t + 1);
        });
        wait_tiles();   // key image t + 1 and score image t + 2
        ring_barrier();
    }
    // Copies issued past the last tile may still be landing in ring buffers that the solve
    // area overlaps: wait for this wave's loads (the barrier below covers the others).
    __builtin_amdgcn_s_waitcnt(0x0 | (0x7 << 4) | (0xF << 8));
    LDS_FENCE();

    // ---- block sums -> LDS (outside the solve area)
    float* skm = reinterpret_cast<float*>(smem + K8_MEAN_OFF);   // [query][feature]
    float* omp = skm + K8_BQ * D8;                                // [scoring wave][query]
    om2p += __shfl_xor(om2p, 16);
    om2p += __shfl_xor(om2p, 32);
#pragma unroll
    for (int r = 0; r < 4; ++r)
        if (4 * g + r < K8_BQ) skm[(4 * g + r) * D8 + 16 * w + c] = sk[r];
    if (scorer && g == 0 && colv) omp[w * 16 + c] = om2p;
    __syncthreads();

    // ---- the wave's solve; row layout: lane holds rows lane and lane + 64.
    // z = kbar - q with kbar = a + S_k / omega'.
    float* Sg = reinterpret_cast<float*>(smem) + w * S8_FLOATS;
    const float* anc = anchors + static_cast<int64_t>(bh) * 2 * D8;
    const int iq = i0 + wu;
    const int iqc = min(iq, n - 1);
    float om2 = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t) om2 += omp[t * 16 + wu];
    const float iom2 = 1.0f / om2;   // >= 1: the query's top-scoring key has weight 1
    const float* skq = skm + wu * D8;
    const float lam = lambda * exp2f(-mrow[static_cast<int64_t>(bh) * prows + (iqc - row0)]);
    float z[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int a = lane + 64 * h;
        z[h] = fmaf(skq[a], iom2, anc[a]) - bf16_bits_to_f32(q[base + static_cast<int64_t>(iqc) * D8 + a]);
    }
    // lambda > 0: drop only pivots that rounding made non-positive; lambda = 0: also drop
    // directions the prefix leaves (numerically) undetermined, below 1e-6 of the largest
    // diagonal entry of the downdated matrix.
    float thr = 0.0f;
    if (!(lambda > 0.0f)) {
        float dmax = -INFINITY;
#pragma unroll
        for (int I = 0; I < 8; ++I)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (4 * g + r == c) {
                    const float sv = skq[16 * I + c];
                    dmax = fmaxf(dmax, ckk[ub8(I, I)][r] - sv * sv * iom2 + lam);
                }
        thr = 1e-6f * wave_max8(dmax);
    }
    // The check's key scale: trace of sum R R^T (before the downdate) / omega'.
    float tr = 0.0f;
#pragma unroll
    for (int I = 0; I < 8; ++I)
#pragma unroll
        for (int r = 0; r < 4; ++r) tr += 4 * g + r == c ? ckk[ub8(I, I)][r] : 0.0f;
    tr = wave_sum8(tr);
    float yd[8];
    float dropped = 0.0f;
    solve8(ckk, z, thr, lam, iom2, skq, Sg, yd, dropped, lane, g, c);
    // Check target: the LLA weights applied to the centred keys give q - a + lambda e^{-m} y
    // (for the y they were formed with); its projections on directions t = 8 g + tt, the
    // sign of feature f = 16 J + c being (-1)^popcount(f & (4t + 1)).
    float cv[8];
#pragma unroll
    for (int J = 0; J < 8; ++J) {
        const int a = 16 * J + c;
        cv[J] = bf16_bits_to_f32(q[base + static_cast<int64_t>(iqc) * D8 + a]) - anc[a] + lam * yd[J];
    }
    float chk_c = 0.0f;   // direction 8 g + c, for lanes c < 8
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
        const int ml = chk8_mask(tt) & 15, mh = 2 * g + (tt >= 4 ? 1 : 0);   // bits of 4 (8g + tt) + 1
        const bool sl = (__builtin_popcount(c & ml) & 1) != 0;
        float part = 0.0f;
#pragma unroll
        for (int J = 0; J < 8; ++J) {
            const bool sj = (__builtin_popcount(J & mh) & 1) != 0;
            part += (sl != sj) ? -cv[J] : cv[J];
        }
        const float sum = row_sum8(part);
        chk_c = c == tt ? sum : chk_c;
    }
    LDS_FENCE();
    // yh 2^e with max |.| in [2^13, 2^14), as fp16 hi + lo (about 22 bits together), and
    // gamma = 1 + S_k . yh / omega'.  Lane (g, c) holds rows 16 J + c; lanes g = 0 store.
    float amax = 0.0f;
#pragma unroll
    for (int J = 0; J < 8; ++J) amax = fmaxf(amax, fabsf(yd[J] * om2));
    amax = wave_max8(amax);
    int ex = 0;
    (void)frexpf(amax, &ex);
    ex = max(ex, -100);   // keeps 2^(14 - ex) finite
    const float sig = amax > 0.0f ? ldexpf(1.0f, 14 - ex) : 1.0f;
    _Float16 hi[8], lo[8];
    float dot = 0.0f;
#pragma unroll
    for (int J = 0; J < 8; ++J) {
        const float ys = (yd[J] * om2) * sig;
        hi[J] = static_cast<_Float16>(ys);
        lo[J] = static_cast<_Float16>(ys - static_cast<float>(hi[J]));
        dot = fmaf(skq[16 * J + c], static_cast<float>(hi[J]) + static_cast<float>(lo[J]), dot);
    }
    dot = wave_sum8(dot) * 0.25f;   // every row of 16 lanes holds the same 128 products
    if (iq < n && g == 0) {
        const int64_t qrow = static_cast<int64_t>(bh) * prows + (iq - row0);
#pragma unroll
        for (int J = 0; J < 8; ++J) {
            yhl[qrow * P8_YLD + 16 * J + c] = hi[J];
            yhl[qrow * P8_YLD + D8 + 16 * J + c] = lo[J];
        }
        // qsc[3] flags a pivot dropped although the ridge keeps the system positive definite.
        if (c == 0) {
            *reinterpret_cast<float4v*>(qsc + qrow * P8_QSC) =
                float4v{fmaf(dot / sig, iom2, 1.0f), 1.0f / sig, iom2, lambda > 0.0f ? dropped : 0.0f};
            *reinterpret_cast<float4v*>(qsc + qrow * P8_QSC + 4) = float4v{tr * iom2, 0.0f, 0.0f, 0.0f};
        }
    }
    if (iq < n && c < 8) chk[(static_cast<int64_t>(bh) * prows + (iq - row0)) * P8_CHK + 8 * g + c] = chk_c;
}

// ---------------------------------------------------------------------------------------
// Probe pass (rows i >= row0): b_i = a_v + (1/omega') sum_j P_ij (v_j - a_v) with
// P_ij = fp16(w_ij fp16(gamma_i - (k_j - a).yh_i 2^-e)).  Block = 4 waves x 2 sets of 16
// queries (the sets share the key and value operands), one block per CU; each 64-key tile
// (bf16 keys and fp16 centred keys key-major, fp16 centred values feature-major: 52 KiB) is
// copied into one of two LDS buffers while the other is in use.  Per tile, wave and set, per
// 16-key block: S^T = K Q^T (bf16 MFMAs, the key-moment kernel's operands in its order, so
// bitwise its scores and weights), U^T = (K - a)(yh_hi + yh_lo)^T (fp16 MFMAs); lane (g, c)
// register r holds key 16 kb + 4 g + r of query c, already the A operand of O += P (V - a_v)
// over 32-key steps.
constexpr int P8_SETS = 2, P8_QW = 16 * P8_SETS, P8_QB = NW8 * P8_QW;
constexpr int P8_BUF = KM_STRIDE8 + F_BYTES + KU_TILE_BYTES;   // bf16 K | fp16 K - a | fp16 V - a_v | check image
constexpr int P8_LOADS = P8_BUF / 1024;                // 57
constexpr int P8_WLOADS = (P8_LOADS + NW8 - 1) / NW8;  // 15 (the surplus repeat the last chunk)
constexpr int P8_SMEM = 2 * P8_BUF;


__global__ __launch_bounds__(256, 1) void lla8_probe_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ mrow, const float* __restrict__ anchors,
    const unsigned char* __restrict__ km, const unsigned char* __restrict__ vf,
    const unsigned char* __restrict__ kuf, const _Float16* __restrict__ yhl, const float* __restrict__ qsc,
    const float* __restrict__ chk, float* __restrict__ out, unsigned* __restrict__ guard, int* __restrict__ list,
    int n, int row0, int BH, float sl2) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int g = lane >> 4, c = lane & 15;
    const int prows = n - row0;
    const int nblk = (prows + P8_QB - 1) / P8_QB;
    int blk, bh;
    head_major_block(static_cast<int>(blockIdx.x), BH, nblk, &bh, &blk);
    const int i0 = row0 + blk * P8_QB;
    const int qw0 = i0 + P8_QW * wu;
    const int wave_last = min(qw0 + P8_QW - 1, n - 1);
    const int block_last = min(i0 + P8_QB - 1, n - 1);
    const int64_t base = static_cast<int64_t>(bh) * n * D8;
    if (head_unsafe(guard, bh)) {   // block-uniform: the head's rows go to the fp64 kernel
#pragma unroll
        for (int st = 0; st < P8_SETS; ++st)
            if (g == 0 && qw0 + 16 * st + c < n) hand_back(guard, list, bh, n, qw0 + 16 * st + c);
        return;
    }

    bf16x8 qf[P8_SETS][4];
    half8 yh[P8_SETS][4], yl[P8_SETS][4];
    float gam[P8_SETS], isig[P8_SETS], hm[P8_SETS];
    int qc[P8_SETS];
#pragma unroll
    for (int st = 0; st < P8_SETS; ++st) {
        qc[st] = min(qw0 + 16 * st + c, n - 1);
        const int64_t qrow = static_cast<int64_t>(bh) * prows + (qc[st] - row0);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            qf[st][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(
                                                        q + base + static_cast<int64_t>(qc[st]) * D8 + 32 * ks + 8 * g));
            yh[st][ks] = *reinterpret_cast<const half8*>(yhl + qrow * P8_YLD + 32 * ks + 8 * g);
            yl[st][ks] = *reinterpret_cast<const half8*>(yhl + qrow * P8_YLD + D8 + 32 * ks + 8 * g);
        }
        const float4v sc = *reinterpret_cast<const float4v*>(qsc + qrow * P8_QSC);
        gam[st] = sc[0];
        isig[st] = sc[1];
        hm[st] = 0.5f * mrow[qrow];
    }
    const float hs = 0.5f * sl2;

    const int ntiles = block_last / T8 + 1;
    const int ptiles = (n + T8 - 1) / T8;
    const __amdgpu_buffer_rsrc_t kres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(uniform_ptr(km + static_cast<int64_t>(bh) * ptiles * KM_STRIDE8)), 0,
        ptiles * KM_STRIDE8, 0x00020000);
    const __amdgpu_buffer_rsrc_t vres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(uniform_ptr(vf + static_cast<int64_t>(bh) * ptiles * F_BYTES)), 0,
        ptiles * F_BYTES, 0x00020000);
    const __amdgpu_buffer_rsrc_t ures = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(uniform_ptr(kuf + static_cast<int64_t>(bh) * ptiles * KU_TILE_BYTES)), 0,
        ptiles * KU_TILE_BYTES, 0x00020000);
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem));
    // Chunk u of a buffer: u < 34 from the key-major images, u < 52 from the value image, the
    // rest from the check image.  Wave w issues chunks w, w + 4, ... (clamped to the last).
    constexpr int U_KM = KM_STRIDE8 / 1024, U_V = U_KM + F_BYTES / 1024;
    auto issue = [&](int tt) {
        const int ts = min(tt, ntiles - 1);
        const uint32_t dst = lds0 + static_cast<uint32_t>((tt % 2) * P8_BUF);
#pragma unroll
        for (int e = 0; e < P8_WLOADS; ++e) {
            const int u = min(wu + NW8 * e, P8_LOADS - 1);
            auto* ldst = reinterpret_cast<__attribute__((address_space(3))) void*>(static_cast<uintptr_t>(dst + u * 1024));
            if (u < U_KM)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(kres, ldst, 16, lane * 16 + u * 1024, ts * KM_STRIDE8, 0, 0);
            else if (u < U_V)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(vres, ldst, 16, lane * 16 + (u - U_KM) * 1024, ts * F_BYTES, 0, 0);
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

    float4v o[P8_SETS][8], ok[P8_SETS][NCHK / 16];
    float wvn[P8_SETS];   // sum w |v - a_v|^2 of query c over this lane's keys
#pragma unroll
    for (int st = 0; st < P8_SETS; ++st) {
#pragma unroll
        for (int fv = 0; fv < 8; ++fv) o[st][fv] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < NCHK / 16; ++db) ok[st][db] = float4v{0.f, 0.f, 0.f, 0.f};
        wvn[st] = 0.0f;
    }
    issue(0);
    wait_and_sync();
    auto tile_step = [&](const int t, auto phase) {
        issue(t + 1);   // into the buffer tile t-1 used
        const int j0 = t * T8;
        auto tile_body = [&](auto masked) {
            const unsigned char* cur = smem + (t % 2) * P8_BUF;
            const unsigned char* KB = cur;
            const unsigned char* KC = cur + KM_BYTES;
            const _Float16* VI = reinterpret_cast<const _Float16*>(cur + KM_STRIDE8);
            const _Float16* UI = reinterpret_cast<const _Float16*>(cur + KM_STRIDE8 + F_BYTES);
            const float* NR = reinterpret_cast<const float*>(cur + KM_STRIDE8 + F_BYTES + KU8_NRM);
            half4 p[P8_SETS][4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int ro = (kb * 16 + c) * (K_LD * 2) + 16 * g;
                bf16x8 kk[4];
                half8 kc[4];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    kk[ks] = *reinterpret_cast<const bf16x8*>(KB + ro + 64 * ks);
                    kc[ks] = *reinterpret_cast<const half8*>(KC + ro + 64 * ks);
                }
#pragma unroll
                for (int st = 0; st < P8_SETS; ++st) {
                    float4v sv = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) sv = mfma_bf16(kk[ks], qf[st][ks], sv);
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) u = mfma_f16(kc[ks], yh[st][ks], u);
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) u = mfma_f16(kc[ks], yl[st][ks], u);
                    const bool full = !decltype(masked)::value || j0 + T8 - 1 <= qw0 + 16 * st;
                    half4 sw4, t4;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float e = __builtin_amdgcn_exp2f(fmaf(sv[r], hs, -hm[st]));
                        if (!full) e = j0 + kb * 16 + 4 * g + r <= qc[st] ? e : 0.0f;
                        sw4[r] = static_cast<_Float16>(e);
                        t4[r] = static_cast<_Float16>(fmaf(-u[r], isig[st], gam[st]));
                    }
                    const half4 w4 = sw4 * sw4;   // w = fp16(sw^2) as in the key-moment kernel
                    p[st][kb] = w4 * t4;          // then fp16(w t)
                    const float4v nr = *reinterpret_cast<const float4v*>(NR + kb * 16 + 4 * g);
#pragma unroll
                    for (int r = 0; r < 4; ++r) wvn[st] = fmaf(static_cast<float>(w4[r]), nr[r], wvn[st]);
                }
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int fv = 0; fv < 8; ++fv) {
                    const half8 vb = *reinterpret_cast<const half8*>(VI + (fv * 16 + c) * F_LD + 32 * ks + 8 * g);
#pragma unroll
                    for (int st = 0; st < P8_SETS; ++st) {
                        const half8 pa = __builtin_shufflevector(p[st][2 * ks], p[st][2 * ks + 1], 0, 1, 2, 3, 4, 5, 6, 7);
                        o[st][fv] = mfma_f16(pa, vb, o[st][fv]);
                    }
                }
#pragma unroll
                for (int db = 0; db < NCHK / 16; ++db) {
                    const half8 ub = *reinterpret_cast<const half8*>(UI + (db * 16 + c) * F_LD + 32 * ks + 8 * g);
#pragma unroll
                    for (int st = 0; st < P8_SETS; ++st) {
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
    // Tiles wholly below the wave's first query need no causal mask: they run first, in a
    // loop of their own with the unmasked body.
    const int tfull = min(ntiles, (qw0 + 1) / T8);
    for (int t = 0; t < tfull; ++t) tile_step(t, std::false_type{});
    for (int t = tfull; t < ntiles; ++t) tile_step(t, std::true_type{});
    __builtin_amdgcn_s_waitcnt(0x0 | (0x7 << 4) | (0xF << 8));   // copies past the last tile

    // Output rows: lane (g, c) register r of set st = query qw0 + 16 st + 4 g + r, feature 16 fv + c
    // (direction 16 db + c of the check sums).  A row goes to the fp64 kernel if its output is
    // not finite, its solve dropped a pivot (qsc[3]), or its check exceeds CHK_TOL: the
    // projected deviation of sum_j P_ij (k_j - a) / omega' from q - a + lambda e^{-m} y, in
    // units of the weighted rms |k - a|, times the weighted rms |v - a_v| over |b|.
    const float* anc = anchors + static_cast<int64_t>(bh) * 2 * D8 + D8;
#pragma unroll
    for (int st = 0; st < P8_SETS; ++st) {
        float vq = wvn[st];   // sum_j w_j |v_j - a_v|^2 of query c, then of query 4 g + r below
        vq += __shfl_xor(vq, 16);
        vq += __shfl_xor(vq, 32);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = qw0 + 16 * st + 4 * g + r;
            const int64_t qrow = static_cast<int64_t>(bh) * prows + (min(i, n - 1) - row0);
            const float4v sc = *reinterpret_cast<const float4v*>(qsc + qrow * P8_QSC);
            const float kn2 = qsc[qrow * P8_QSC + 4];
            float bb = 0.0f, rr = 0.0f;
#pragma unroll
            for (int fv = 0; fv < 8; ++fv) {
                const float ov = fmaf(o[st][fv][r], sc[2], anc[fv * 16 + c]);
                bb = fmaf(ov, ov, bb);
                if (i < n) out[base + static_cast<int64_t>(i) * D8 + fv * 16 + c] = ov;
            }
#pragma unroll
            for (int db = 0; db < NCHK / 16; ++db) {
                const float dv = fmaf(ok[st][db][r], sc[2], -chk[qrow * P8_CHK + 16 * db + c]);
                rr = fmaf(dv, dv, rr);
            }
            bb = row_sum8(bb);
            rr = row_sum8(rr);
            const float vn2 = __shfl(vq, 4 * g + r) * sc[2];
            const float est2 = (rr * (1.0f / NCHK)) * vn2 / (kn2 * bb);
            const bool bad = i < n && (!(est2 <= CHK_TOL * CHK_TOL) || sc[3] != 0.0f);
            const uint64_t badm = __ballot(bad);   // every lane takes part
            if (c == 0 && i < n && ((badm >> (16 * g)) & 0xFFFFull) != 0) hand_back(guard, list, bh, n, i);
        }
    }
}

// Rows [0, 4d): the fp64 kernel; rows [4d, n): this path.
int fast8_row0(int64_t n) { return static_cast<int>(n < 4 * D8 ? n : 4 * D8); }

// Workspace, each region 256-byte aligned: row maxima [B*H][n - 4d] | anchor partial sums
// [B*H][16][2d] | anchors [B*H][2d] | K feature-major images [B*H][tiles] | V feature-major
// images [B*H][tiles] | key-major images (bf16, centred fp16) [B*H][tiles] | check images
// [B*H][tiles] | probe solutions (fp16 hi, lo) [B*H][n - 4d][2d] | probe scalars
// [B*H][n - 4d][8] | check targets [B*H][n - 4d][32] | guard: count of rows handed back,
// then per head the largest |k - a| and |v - a_v| (float bits) [1 + 2 B*H] | rows handed
// back [B*H][n - 4d].
struct Fast8Layout {
    int64_t mrow, partial, anchors, kf, vf, km, kuf, yhl, qsc, chk, guard, list, total;
};

Fast8Layout fast8_layout(int64_t BH, int64_t n) {
    auto up = [](int64_t bytes) { return (bytes + 255) & ~int64_t(255); };
    const int64_t prows = n - fast8_row0(n), tiles = (n + T8 - 1) / T8;
    Fast8Layout L;
    L.mrow = 0;
    L.partial = L.mrow + up(BH * prows * 4);
    L.anchors = L.partial + up(BH * A8_SLICES * 2 * D8 * 4);
    L.kf = L.anchors + up(BH * 2 * D8 * 4);
    L.vf = L.kf + BH * tiles * F_BYTES;
    L.km = L.vf + BH * tiles * F_BYTES;
    L.kuf = L.km + BH * tiles * KM_STRIDE8;
    L.yhl = L.kuf + BH * tiles * KU_TILE_BYTES;
    L.qsc = L.yhl + up(BH * prows * P8_YLD * 2);
    L.chk = L.qsc + up(BH * prows * P8_QSC * 4);
    L.guard = L.chk + up(BH * prows * P8_CHK * 4);
    L.list = L.guard + up((1 + 2 * BH) * 4);
    L.total = L.list + up(BH * prows * 4);
    return L;
}

// Dynamic-LDS limits are set per device, the first time a device launches this path.
std::mutex g_attr8_mu;
bool g_attr8_done[64] = {};

hipError_t ensure_attributes8() {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_attr8_mu);
    if (g_attr8_done[dev]) return hipSuccess;
    if ((err = hipFuncSetAttribute(reinterpret_cast<const void*>(&lla8_keymom_kernel),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, K8_SMEM)) != hipSuccess)
        return err;
    if ((err = hipFuncSetAttribute(reinterpret_cast<const void*>(&lla8_probe_kernel),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, P8_SMEM)) != hipSuccess)
        return err;
    g_attr8_done[dev] = true;
    return hipSuccess;
}

}  // namespace

size_t fast128_workspace_bytes(int64_t B, int64_t H, int64_t n) {
    if (n - fast8_row0(n) <= 0) return 0;
    return static_cast<size_t>(fast8_layout(B * H, n).total);
}

int64_t fast128_fallback_count_offset(int64_t B, int64_t H, int64_t n) {
    if (n - fast8_row0(n) <= 0) return -1;
    return fast8_layout(B * H, n).guard;
}

hipError_t launch_fast128(const Problem& p, void* workspace) {
    hipError_t err;
    const int n = static_cast<int>(p.n);
    const int BH = static_cast<int>(p.B * p.H);
    const int row0 = fast8_row0(p.n);
    if ((err = launch_short128(p, row0)) != hipSuccess) return err;
    if (n <= row0) return hipSuccess;
    if ((err = ensure_attributes8()) != hipSuccess) return err;
    const float sl2 = static_cast<float>(LOG2E / p.h);
    const auto* q = static_cast<const uint16_t*>(p.q);
    const auto* k = static_cast<const uint16_t*>(p.k);
    const auto* v = static_cast<const uint16_t*>(p.v);
    const Fast8Layout L = fast8_layout(BH, n);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    float* mrow = reinterpret_cast<float*>(ws + L.mrow);
    float* partial = reinterpret_cast<float*>(ws + L.partial);
    float* anchors = reinterpret_cast<float*>(ws + L.anchors);
    unsigned char* kf = ws + L.kf;
    unsigned char* vf = ws + L.vf;
    unsigned char* km = ws + L.km;
    _Float16* yhl = reinterpret_cast<_Float16*>(ws + L.yhl);
    float* qsc = reinterpret_cast<float*>(ws + L.qsc);
    float* chk = reinterpret_cast<float*>(ws + L.chk);
    unsigned char* kuf = ws + L.kuf;
    unsigned* guard = reinterpret_cast<unsigned*>(ws + L.guard);
    int* list = reinterpret_cast<int*>(ws + L.list);
    const int ptiles = (n + T8 - 1) / T8;
    const int prows = n - row0;
    prof_begin(p.stream, "lla8_anchor_kernel");
    lla8_anchor_kernel<<<dim3(static_cast<unsigned>(BH) * A8_SLICES), dim3(256), 0, p.stream>>>(k, v, partial, guard,
                                                                                              n);
    prof_end(p.stream);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    prof_begin(p.stream, "lla8_pack_kernel");
    lla8_pack_kernel<<<dim3(static_cast<unsigned>(BH) * ptiles), dim3(256), 0, p.stream>>>(k, v, partial, anchors, kf,
                                                                                           vf, km, kuf, guard, n,
                                                                                           ptiles);
    prof_end(p.stream);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    prof_begin(p.stream, "lla8_rowmax_kernel");
    lla8_rowmax_kernel<<<dim3(static_cast<unsigned>(BH) * ((prows + R8_QB - 1) / R8_QB)), dim3(256), 0, p.stream>>>(
        q, km, mrow, n, row0, BH, sl2);
    prof_end(p.stream);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    prof_begin(p.stream, "lla8_keymom_kernel");
    lla8_keymom_kernel<<<dim3(static_cast<unsigned>(BH) * ((prows + K8_BQ - 1) / K8_BQ)), dim3(KW8 * 64), K8_SMEM,
                         p.stream>>>(q, mrow, anchors, kf, km, yhl, qsc, chk, guard, n, row0, BH, sl2,
                                     static_cast<float>(p.lambda));
    prof_end(p.stream);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    prof_begin(p.stream, "lla8_probe_kernel");
    lla8_probe_kernel<<<dim3(static_cast<unsigned>(BH) * ((prows + P8_QB - 1) / P8_QB)), dim3(256), P8_SMEM,
                        p.stream>>>(q, mrow, anchors, km, vf, kuf, yhl, qsc, chk, p.out, guard, list, n, row0, BH,
                                    sl2);
    prof_end(p.stream);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    // Rows handed back by the range and finiteness checks, in fp64.
    const int cap = BH * prows;
    return launch_exact_list(p, list, reinterpret_cast<const int*>(guard), cap < 2048 ? cap : 2048);
}

}  // namespace lla
