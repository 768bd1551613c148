// Causal Parallax forward with a caller-supplied probe rho:
//
//   o_i = vbar_i - Sigma_KV^(i) rho_i,   p_ij = softmax_j(q_i . k_j / h), j <= i,
//   vbar_i = E_p[v],  Sigma_KV^(i) = E_p[(v - vbar_i)(k - kbar_i)^T]
//
// ("Parallax" blog post, section 2 "Additive Correction to Softmax" and "Parallax": the
// additive form of LLA with the boundary factor eta set to 0 and the probe given instead of
// solved; Appendix B derives the additive form.)
//
// Matrix-core path (bf16 inputs, d = 64): the two-branch form of the blog's section 3 "One
// extra branch, no extra I/O": the softmax branch keeps d1 = sum P1, O1 = sum P1 v with
// P1 = exp(s - m); the covariance branch shares m and the tiles, and keeps
// d2 = sum P2, O2 = sum P2 v with P2 = P1 * (rho . k); the result is merged at the end as in
// the blog's Appendix C (item 3):  o = O1/d1 - (O2/d1 - (O1/d1)(d2/d1)).
// Differences from the pages' form, none of which changes the result in exact arithmetic:
//   * the probe scores are centred, s2_j = rho . (k_j - a) with a the head's mean key: a
//     constant shift of s2 cancels in the merge, and centring keeps P2 small, so its fp16
//     rounding error is small;
//   * m is the row's exact maximum, from a first pass over the key tiles (scores only), so
//     P1 <= 1 and the second pass needs no rescaling (a running max with rescaling measured
//     slower: its per-step maximum and test cost more in this loop than the first pass);
//   * s2 is scaled by a per-query power of two sigma that keeps |P2| below 2^14 (P1 <= 1 and
//     |s2| <= |rho| (max_j |k_j| + |a|)), so that P2 fits fp16; the merge divides by it;
//   * P1 and P2 enter the P V products as fp16 (v as fp16, exact for bf16 values in the fp16
//     range); d1 and d2 sum the same rounded values, so the rounding only perturbs weights.
// Range guard: a head whose largest |v| lies outside [2^-10, 2^16) (or is not finite) is left
// to the fp64 row code: fp16 would overflow above, and below, its subnormal spacing 2^-24
// would no longer be negligible against the head's values.  The pack kernel records each
// tile's largest |v|; the streaming kernel's blocks of such a head exit at once and list the
// head; a fallback launch runs the generic row code over the listed heads.
// Generic path (fp32 or bf16, d in {16, 32, 64, 128}): fp64, one block per row.
#include "lla_device.h"
#include "lla_internal.h"

#include <math.h>

#include <type_traits>

namespace lla {
namespace {

constexpr int MT = 64;                       // keys per tile
constexpr int KM_LD = FD + 8;                // key-major bf16 row (halves): 64 features + 8 padding
// Feature-major fp16 row (halves): 64 keys + 4 of padding.  A row is 34 banks, so the 16
// rows that one 8-byte read of 16 lanes touches fall on distinct bank pairs.
constexpr int V_LD = MT + 4;
constexpr int X_KIMG = MT * KM_LD * 2;       // 9 KiB
// Tile image: bf16 K key-major | fp16 V feature-major, padded to whole KiB (the tail unused).
constexpr int X_TILE = (X_KIMG + FD * V_LD * 2 + 1023) / 1024 * 1024;
constexpr int X_WAVES = 4;
constexpr int X_SETS = 2;                    // query sets of 16 per wave
constexpr int X_QW = 16 * X_SETS;
constexpr int X_QB = X_WAVES * X_QW;         // 128 queries per block
constexpr int X_LOADS = X_TILE / 1024;       // wave-wide copies of 16 B per lane per tile
constexpr int X_WLOADS = (X_LOADS + X_WAVES - 1) / X_WAVES;
constexpr int X_NBUF = 3;                    // tile ring: compute t, t+1 landing, t+2 in flight
static_assert(X_TILE % 1024 == 0 && X_KIMG % 1024 == 0, "tile image must be whole wave copies");

__device__ __forceinline__ float wave_max64(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum64(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// Pack K and V of one 64-key tile (zero past n) into the tile image: K key-major as given
// (bf16, rows of KM_LD halves) and V feature-major as fp16 (rows of V_LD halves; exact for
// bf16 values in the fp16 range); also the tile's key sum (per feature) and its largest key
// norm.  Thread -> keys 2p, 2p+1 and features 8fg .. 8fg+7.
__global__ __launch_bounds__(256) void lla_parallax_pack_kernel(const uint16_t* __restrict__ k,
                                                                const uint16_t* __restrict__ v,
                                                                unsigned char* __restrict__ img,
                                                                float* __restrict__ ksum,
                                                                float* __restrict__ kmax,
                                                                float* __restrict__ vmax,
                                                                unsigned* __restrict__ nlisted, int n,
                                                                int ntiles) {
    __shared__ float red[32][FD + 1];
    __shared__ float nrm[8][MT];
    __shared__ float vmw[4];
    // The list of heads left to the fallback starts empty (nothing else of this call has
    // touched it yet; the streaming kernel runs after this one).
    if (blockIdx.x == 0 && threadIdx.x == 0) *nlisted = 0u;
    const int bh = static_cast<int>(blockIdx.x) / ntiles, t = static_cast<int>(blockIdx.x) % ntiles;
    const int tid = threadIdx.x, pr = tid & 31, fg = tid >> 5;
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
    unsigned char* ti = img + (static_cast<int64_t>(bh) * ntiles + t) * X_TILE;
    *reinterpret_cast<uint4*>(ti + (2 * pr) * (KM_LD * 2) + 16 * fg) = k0;
    *reinterpret_cast<uint4*>(ti + (2 * pr + 1) * (KM_LD * 2) + 16 * fg) = k1;
    if (fg == 0) {
        *reinterpret_cast<uint4*>(ti + (2 * pr) * (KM_LD * 2) + 2 * FD) = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(ti + (2 * pr + 1) * (KM_LD * 2) + 2 * FD) = make_uint4(0, 0, 0, 0);
    }
    uint32_t* vd = reinterpret_cast<uint32_t*>(ti + X_KIMG);
    const uint32_t ka[4] = {k0.x, k0.y, k0.z, k0.w}, kb[4] = {k1.x, k1.y, k1.z, k1.w};
    const uint32_t va[4] = {v0.x, v0.y, v0.z, v0.w}, vb[4] = {v1.x, v1.y, v1.z, v1.w};
    float na = 0.0f, nb = 0.0f, vm = 0.0f;   // vm: largest |v| of this thread (a NaN counts as inf)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int row = 8 * fg + e, hi = e & 1;
        const float xa = __uint_as_float(hi ? (ka[e >> 1] & 0xffff0000u) : (ka[e >> 1] << 16));
        const float xb = __uint_as_float(hi ? (kb[e >> 1] & 0xffff0000u) : (kb[e >> 1] << 16));
        red[pr][row] = xa + xb;
        na = fmaf(xa, xa, na);
        nb = fmaf(xb, xb, nb);
        const float ya = __uint_as_float(hi ? (va[e >> 1] & 0xffff0000u) : (va[e >> 1] << 16));
        const float yb = __uint_as_float(hi ? (vb[e >> 1] & 0xffff0000u) : (vb[e >> 1] << 16));
        vm = fmaxf(vm, ya == ya ? fabsf(ya) : INFINITY);
        vm = fmaxf(vm, yb == yb ? fabsf(yb) : INFINITY);
        h16x2 vv;
        vv[0] = static_cast<_Float16>(ya);
        vv[1] = static_cast<_Float16>(yb);
        vd[row * (V_LD / 2) + pr] = __builtin_bit_cast(uint32_t, vv);
        if (pr < (V_LD - MT) / 2) vd[row * (V_LD / 2) + MT / 2 + pr] = 0u;   // row padding
    }
    nrm[fg][2 * pr] = na;
    nrm[fg][2 * pr + 1] = nb;
    vm = wave_max64(vm);
    if ((tid & 63) == 0) vmw[tid >> 6] = vm;
    __syncthreads();
    const int64_t tix = static_cast<int64_t>(bh) * ntiles + t;
    if (tid == 0) vmax[tix] = fmaxf(fmaxf(vmw[0], vmw[1]), fmaxf(vmw[2], vmw[3]));
    if (tid < FD) {
        float s = 0.0f;
        for (int p = 0; p < 32; ++p) s += red[p][tid];
        ksum[tix * FD + tid] = s;
        float sq = 0.0f;
#pragma unroll
        for (int f = 0; f < 8; ++f) sq += nrm[f][tid];
        const float mx = wave_max64(sqrtf(sq));
        if (tid == 0) kmax[tix] = mx;
    }
}

// The streaming pass.  Block = 4 waves x 32 queries (two sets of 16 per wave, which share
// the key and value operands), two blocks per CU; each tile image is copied straight into
// a ring of three LDS buffers, two tiles ahead of the one in use.  Per tile, wave and query set:
// the tile in two steps of 32 keys:
//   S1^T = K Q^T and S2^T = K R^T (bf16 MFMA pairs, one K operand for both), lane (g, c)
//   register r = key 16 kb + 4g + r of query c;
//   the step's max of S1 over the query's keys -> running max, rescale of (d1, d2, O1, O2)
//   by alpha = 2^(m_old - m_new) when it grows (steps of 32 rather than whole tiles keep the
//   scores of a step, not of a tile, beside the accumulators: two waves per SIMD);
//   P1 = fp16(2^(s1 log2e/h - m)), P2 = fp16(P1 (s2 - rho.a) sigma);
//   O^T += V^T P^T (fp16 MFMA, V the A operand), so that lane (g, c) register r of O holds
//   feature 16 fv + 4g + r of query c -- the same query as the lane's row statistics.
template <bool kStats>   // kStats: also write the per-row statistics the backward reads
__global__ __launch_bounds__(X_WAVES * 64, 2) void lla_parallax_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ rho, const unsigned char* __restrict__ img,
    const float* __restrict__ ksum, const float* __restrict__ kmax, const float* __restrict__ vmax,
    unsigned* __restrict__ nlisted, int* __restrict__ hlist, float* __restrict__ out,
    float* __restrict__ stats, int n, int BH, float sl2) {
    __shared__ __attribute__((aligned(16))) unsigned char ring[X_NBUF * X_TILE];
    __shared__ float akm[FD];
    __shared__ float kbound;
    __shared__ int vout;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int g = lane >> 4, c = lane & 15;
    const int nblk = (n + X_QB - 1) / X_QB;
    int blk, bh;
    head_major_block(static_cast<int>(blockIdx.x), BH, nblk, &bh, &blk);
    const int i0 = blk * X_QB;
    const int qw0 = i0 + X_QW * wu;                   // this wave's first query
    const int wave_last = min(qw0 + X_QW - 1, n - 1);
    const int block_last = min(i0 + X_QB - 1, n - 1);
    const int64_t base = static_cast<int64_t>(bh) * n * FD;
    const int ptiles = (n + MT - 1) / MT;
    const int ntiles = block_last / MT + 1;

    // Head anchor a = mean key, and max_j |k_j| (wave 1).
    if (wu == 0) {
        float s = 0.0f;
        for (int t = 0; t < ptiles; ++t) s += ksum[(static_cast<int64_t>(bh) * ptiles + t) * FD + lane];
        akm[lane] = s / static_cast<float>(n);
    } else if (wu == 1) {
        float mx = 0.0f;
        for (int t = lane; t < ptiles; t += 64) mx = fmaxf(mx, kmax[static_cast<int64_t>(bh) * ptiles + t]);
        mx = wave_max64(mx);
        if (lane == 0) kbound = mx;
    } else if (wu == 2) {
        // Range guard: the head's largest |v| must lie in [2^-10, 2^16) (or be 0: all values 0).
        float mx = 0.0f;
        for (int t = lane; t < ptiles; t += 64) mx = fmaxf(mx, vmax[static_cast<int64_t>(bh) * ptiles + t]);
        mx = wave_max64(mx);
        if (lane == 0) vout = !(mx < 65536.0f) || (mx > 0.0f && mx < 0x1p-10f);
    }
    __syncthreads();
    if (vout) {   // block-uniform: the head goes to the fallback, listed once (by its first block)
        if (blk == 0 && tid == 0) hlist[atomicAdd(nlisted, 1u)] = bh;
        return;
    }
    const float anorm = sqrtf(wave_sum64(akm[lane] * akm[lane]));
    const float rbound = kbound + anorm;   // >= |k_j - a| for every key of the head

    // Query set st: column c is query qw0 + 16 st + c (clamped to n - 1).
    bf16x8 qf[X_SETS][2], rf[X_SETS][2];
    float csg[X_SETS], sg[X_SETS];   // per query: -(rho . a) sigma and sigma
    int qc[X_SETS];
#pragma unroll
    for (int st = 0; st < X_SETS; ++st) {
        qc[st] = min(qw0 + 16 * st + c, n - 1);
        float pd = 0.0f, pn = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int64_t off = base + static_cast<int64_t>(qc[st]) * FD + 32 * ks + 8 * g;
            const uint4 qr = *reinterpret_cast<const uint4*>(q + off);
            const uint4 rr = *reinterpret_cast<const uint4*>(rho + off);
            qf[st][ks] = __builtin_bit_cast(bf16x8, qr);
            const uint32_t rw[4] = {rr.x, rr.y, rr.z, rr.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float r = __uint_as_float((e & 1) ? (rw[e >> 1] & 0xffff0000u) : (rw[e >> 1] << 16));
                pd = fmaf(r, akm[32 * ks + 8 * g + e], pd);
                pn = fmaf(r, r, pn);
            }
        }
        pd += __shfl_xor(pd, 16);
        pd += __shfl_xor(pd, 32);
        pn += __shfl_xor(pn, 16);
        pn += __shfl_xor(pn, 32);
        // sigma = 2^(14 - e) with |rho| rbound = f 2^e, f in [0.5, 1): P1 <= 1 and
        // |s2 - rho.a| sigma < 2^14, so |P2| < 2^14.
        const float bound = sqrtf(pn) * rbound;
        int ex = 0;
        (void)frexpf(bound, &ex);
        ex = min(max(ex, -100), 100);
        sg[st] = (bound > 0.0f && bound < INFINITY) ? ldexpf(1.0f, 14 - ex) : 1.0f;
        csg[st] = -pd * sg[st];   // -(rho . a) sigma: the initial value of the probe-score sums
        // The probe operand carries sigma: a power of two, exact in bf16.
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const uint4 rr = *reinterpret_cast<const uint4*>(rho + base + static_cast<int64_t>(qc[st]) * FD + 32 * ks + 8 * g);
            const uint32_t rw[4] = {rr.x, rr.y, rr.z, rr.w};
            bf16x8 sc;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                sc[e] = static_cast<__bf16>(sg[st] * __uint_as_float((e & 1) ? (rw[e >> 1] & 0xffff0000u)
                                                                              : (rw[e >> 1] << 16)));
            rf[st][ks] = sc;
        }
    }

    const __amdgpu_buffer_rsrc_t ires = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(uniform_ptr(img + static_cast<int64_t>(bh) * ptiles * X_TILE)), 0,
        ptiles * X_TILE, 0x00020000);
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ring));
    // Tile tt -> buffer tt % 3; wave w copies KiB chunks w, w+4, ... of the first NCH chunks of
    // the tile image (the surplus ones repeat the last chunk); past the last tile the last one
    // is re-read into a dead buffer.
    auto issue = [&](auto nch, int tt) {
        constexpr int NCH = decltype(nch)::value, NW = (NCH + X_WAVES - 1) / X_WAVES;
        const int ts = min(tt, ntiles - 1);
        const uint32_t dst = lds0 + static_cast<uint32_t>((tt % X_NBUF) * X_TILE);
#pragma unroll
        for (int e = 0; e < NW; ++e) {
            const int u = min(wu + X_WAVES * e, NCH - 1);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ires, reinterpret_cast<__attribute__((address_space(3))) void*>(static_cast<uintptr_t>(dst + u * 1024)),
                16, lane * 16 + u * 1024, ts * X_TILE, 0, 0);
        }
    };
    // Tile t+1 has landed -- only tile t+2's copies (NW per wave) may still be in flight: they
    // are the only vector loads in the loops -- and every wave is done with the buffer the
    // next copies overwrite.
    auto next_tile = [](auto nch) {
        constexpr int NW = (decltype(nch)::value + X_WAVES - 1) / X_WAVES;
        static_assert(NW < 16, "vmcnt operand is 4 bits here");
        __builtin_amdgcn_s_waitcnt(NW | (0x7 << 4) | (0x0 << 8));
        LDS_FENCE();
        __builtin_amdgcn_s_barrier();
        LDS_FENCE();
    };
    using KeysOnly = std::integral_constant<int, X_KIMG / 1024>;
    using WholeTile = std::integral_constant<int, X_LOADS>;

    // ---- pass 1: row maxima m_i = max_{j <= i} q_i.k_j, keys only.  Lane (g, c) register r of
    // a score block = key 16 kb + 4g + r of query c of the set.
    float mloc[X_SETS] = {-INFINITY, -INFINITY};
    issue(KeysOnly{}, 0);
    issue(KeysOnly{}, 1);
    next_tile(KeysOnly{});
    for (int t = 0; t < ntiles; ++t) {
        issue(KeysOnly{}, t + 2);
        const int j0 = t * MT;
        auto tile_max = [&](auto masked) {
            const unsigned char* cur = ring + (t % X_NBUF) * X_TILE;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int ro = (kb * 16 + c) * (KM_LD * 2) + 16 * g;
                const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(cur + ro);
                const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(cur + ro + 64);
#pragma unroll
                for (int st = 0; st < X_SETS; ++st) {
                    float4v a = {0.f, 0.f, 0.f, 0.f};
                    a = mfma_bf16(k0, qf[st][0], a);
                    a = mfma_bf16(k1, qf[st][1], a);
                    const bool full = !decltype(masked)::value || j0 + MT - 1 <= qw0 + 16 * st;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        mloc[st] = fmaxf(mloc[st], (full || j0 + kb * 16 + 4 * g + r <= qc[st]) ? a[r] : -INFINITY);
                }
            }
        };
        if (j0 + MT - 1 <= qw0) tile_max(std::false_type{});
        else if (j0 <= wave_last) tile_max(std::true_type{});   // wave-uniform
        next_tile(KeysOnly{});
    }
    // Every wave is done with the ring (and its copies have landed) before pass 2 refills it.
    __builtin_amdgcn_s_waitcnt(0x0 | (0x7 << 4) | (0x0 << 8));
    LDS_FENCE();
    __builtin_amdgcn_s_barrier();
    LDS_FENCE();
    float mrow[X_SETS];   // log2 units
#pragma unroll
    for (int st = 0; st < X_SETS; ++st) {
        float m = fmaxf(mloc[st], __shfl_xor(mloc[st], 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        mrow[st] = m * sl2;
    }

    // ---- pass 2: weights P1 = 2^(s1 log2e/h - m) <= 1 and P2 = P1 (s2 - rho.a) sigma, and the
    // sums d1, d2, O1, O2, in two 32-key steps per tile.
    float d1p[X_SETS], d2p[X_SETS];
    float4v o1[X_SETS][4], o2[X_SETS][4];
#pragma unroll
    for (int st = 0; st < X_SETS; ++st) {
        d1p[st] = 0.0f;
        d2p[st] = 0.0f;
#pragma unroll
        for (int fv = 0; fv < 4; ++fv) {
            o1[st][fv] = float4v{0.f, 0.f, 0.f, 0.f};
            o2[st][fv] = float4v{0.f, 0.f, 0.f, 0.f};
        }
    }
    const h16x2 one2 = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
    float4v csv[X_SETS];   // initial value of the probe-score sums
#pragma unroll
    for (int st = 0; st < X_SETS; ++st) csv[st] = float4v{csg[st], csg[st], csg[st], csg[st]};
    issue(WholeTile{}, 0);
    issue(WholeTile{}, 1);
    next_tile(WholeTile{});
    // Every tile a wave takes starts at or below its first query (tiles and waves are aligned
    // to 64 and 32 rows); a tile wholly below the wave's first query needs no causal mask.
    // Those tiles run first, in a loop of their own with the unmasked body, so the
    // accumulators keep one register assignment from tile to tile.
    auto tile_step = [&](const int t, auto phase) {
        issue(WholeTile{}, t + 2);   // into the buffer tile t-1 used
        const int j0 = t * MT;
        auto tile_body = [&](auto masked) {
            const unsigned char* cur = ring + (t % X_NBUF) * X_TILE;
            const _Float16* VI = reinterpret_cast<const _Float16*>(cur + X_KIMG);
            // K-slots of lane group g in step ks: keys 32 ks + 4g.. and 32 ks + 16 + 4g..
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                float4v s1[X_SETS][2], s2[X_SETS][2];
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) {
                    const int ro = ((2 * ks + hb) * 16 + c) * (KM_LD * 2) + 16 * g;
                    const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(cur + ro);
                    const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(cur + ro + 64);
#pragma unroll
                    for (int st = 0; st < X_SETS; ++st) {
                        float4v a = {0.f, 0.f, 0.f, 0.f};
                        a = mfma_bf16(k0, qf[st][0], a);
                        s1[st][hb] = mfma_bf16(k1, qf[st][1], a);   // pass 1's operands and order
                        const float4v b = mfma_bf16(k0, rf[st][0], csv[st]);
                        s2[st][hb] = mfma_bf16(k1, rf[st][1], b);   // (rho . (k - a)) sigma
                    }
                }
                half4 p1[X_SETS][2], p2[X_SETS][2];
#pragma unroll
                for (int st = 0; st < X_SETS; ++st) {
                    const bool full = !decltype(masked)::value || j0 + 32 * ks + 31 <= qw0 + 16 * st;
#pragma unroll
                    for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            float e = __builtin_amdgcn_exp2f(fmaf(s1[st][hb][r], sl2, -mrow[st]));
                            if (!full) e = j0 + (2 * ks + hb) * 16 + 4 * g + r <= qc[st] ? e : 0.0f;
                            p1[st][hb][r] = static_cast<_Float16>(e);
                            p2[st][hb][r] = static_cast<_Float16>(e * s2[st][hb][r]);
                        }
                        d1p[st] = __builtin_amdgcn_fdot2(__builtin_shufflevector(p1[st][hb], p1[st][hb], 0, 1), one2, d1p[st], false);
                        d1p[st] = __builtin_amdgcn_fdot2(__builtin_shufflevector(p1[st][hb], p1[st][hb], 2, 3), one2, d1p[st], false);
                        d2p[st] = __builtin_amdgcn_fdot2(__builtin_shufflevector(p2[st][hb], p2[st][hb], 0, 1), one2, d2p[st], false);
                        d2p[st] = __builtin_amdgcn_fdot2(__builtin_shufflevector(p2[st][hb], p2[st][hb], 2, 3), one2, d2p[st], false);
                    }
                }
#pragma unroll
                for (int fv = 0; fv < 4; ++fv) {
                    const _Float16* vr = VI + (fv * 16 + c) * V_LD + 32 * ks + 4 * g;
                    const half4 va = *reinterpret_cast<const half4*>(vr);
                    const half4 vb = *reinterpret_cast<const half4*>(vr + 16);
                    const half8 vo = __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                    for (int st = 0; st < X_SETS; ++st) {
                        const half8 pa = __builtin_shufflevector(p1[st][0], p1[st][1], 0, 1, 2, 3, 4, 5, 6, 7);
                        const half8 pb = __builtin_shufflevector(p2[st][0], p2[st][1], 0, 1, 2, 3, 4, 5, 6, 7);
                        o1[st][fv] = mfma_f16(vo, pa, o1[st][fv]);
                        o2[st][fv] = mfma_f16(vo, pb, o2[st][fv]);
                    }
                }
            }
        };
        if constexpr (!decltype(phase)::value) tile_body(std::false_type{});
        else if (j0 <= wave_last) tile_body(std::true_type{});   // wave-uniform
        next_tile(WholeTile{});
    };
    const int tfull = min(ntiles, (qw0 + 1) / MT);   // tiles t with t MT + MT - 1 <= qw0
    for (int t = 0; t < tfull; ++t) tile_step(t, std::false_type{});
    for (int t = tfull; t < ntiles; ++t) tile_step(t, std::true_type{});
    // Copies past the last tile are still landing in LDS: let them finish before exit.
    __builtin_amdgcn_s_waitcnt(0x0 | (0x7 << 4) | (0xF << 8));

    // Merge: o = O1/d1 - (O2/d1 - (O1/d1)(d2/d1)) / sigma; lane (g, c) register r of set st
    // is feature 16 fv + 4g + r of query qw0 + 16 st + c.
#pragma unroll
    for (int st = 0; st < X_SETS; ++st) {
        float d1 = d1p[st] + __shfl_xor(d1p[st], 16);
        d1 += __shfl_xor(d1, 32);
        float d2 = d2p[st] + __shfl_xor(d2p[st], 16);
        d2 += __shfl_xor(d2, 32);
        const int i = qw0 + 16 * st + c;
        if (i < n) {
            const float inv = 1.0f / d1, a2 = d2 * inv, isg = 1.0f / sg[st];
            float* orow = out + base + static_cast<int64_t>(i) * FD;
#pragma unroll
            for (int fv = 0; fv < 4; ++fv) {
                float4v res;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float ob = o1[st][fv][r] * inv;
                    res[r] = ob - (o2[st][fv][r] * inv - ob * a2) * isg;
                }
                *reinterpret_cast<float4v*>(orow + 16 * fv + 4 * g) = res;
            }
            if constexpr (kStats) {   // the row's log-sum-exp of the scores, base 2
                if (g == 0) stats[static_cast<int64_t>(bh) * n + i] = mrow[st] + log2f(d1);
            }
        }
    }
}

// ---------------------------------------------------------------------------------------
// Generic path: one block of 256 threads per row i, fp64 after the load, three passes over
// the prefix in chunks of 256 keys: (0) the row max of the scores; (1) omega and the
// weighted key and value means; (2) u_j = w_j rho . (k_j - kbar) and
// o = vbar - sum_j u_j (v_j - vbar) / omega  (= vbar - Sigma_KV rho).

constexpr int G_NT = 256;
constexpr int G_CHK = 256;

// Row i of head bh, by the whole block (every thread calls it with the same i and bh).
template <typename TIn, int D>
__device__ __forceinline__ void parallax_exact_row(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v, const TIn* __restrict__ rho,
    float* __restrict__ out, float* __restrict__ stats, int n, double inv_h, int i, int bh) {
    constexpr int KL = G_NT / D;   // key lanes of the per-feature sums
    __shared__ double qs[D], rs[D], kbar[D], vbar[D];
    __shared__ double ws[G_CHK];
    __shared__ double red[G_NT];
    const int tid = threadIdx.x;
    const int64_t base = static_cast<int64_t>(bh) * n * D;
    const int cnt = i + 1;
    for (int e = tid; e < D; e += G_NT) {
        qs[e] = load_f64(q + base, static_cast<int64_t>(i) * D + e);
        rs[e] = load_f64(rho + base, static_cast<int64_t>(i) * D + e);
    }
    __syncthreads();
    auto score = [&](int j) {
        double s = 0.0;
        for (int a = 0; a < D; ++a) s += qs[a] * load_f64(k + base, static_cast<int64_t>(j) * D + a);
        return s * inv_h;
    };
    auto block_reduce = [&](double x, bool is_max) {
        red[tid] = x;
        __syncthreads();
        for (int s = G_NT / 2; s > 0; s >>= 1) {
            if (tid < s) red[tid] = is_max ? fmax(red[tid], red[tid + s]) : red[tid] + red[tid + s];
            __syncthreads();
        }
        const double r = red[0];
        __syncthreads();
        return r;
    };

    // pass 0: row max
    double mloc = -INFINITY;
    for (int j = tid; j < cnt; j += G_NT) mloc = fmax(mloc, score(j));
    const double m = block_reduce(mloc, true);

    // pass 1: omega, kbar, vbar
    const int fa = tid % D, kl = tid / D;
    double acc_w = 0.0, acc_k = 0.0, acc_v = 0.0;
    for (int c0 = 0; c0 < cnt; c0 += G_CHK) {
        const int nk = min(G_CHK, cnt - c0);
        if (tid < nk) ws[tid] = exp(score(c0 + tid) - m);
        __syncthreads();
        for (int jj = kl; jj < nk; jj += KL) {
            const double wj = ws[jj];
            const int64_t off = static_cast<int64_t>(c0 + jj) * D + fa;
            acc_k += wj * load_f64(k + base, off);
            acc_v += wj * load_f64(v + base, off);
        }
        if (tid < nk) acc_w += ws[tid];
        __syncthreads();
    }
    const double omega = block_reduce(acc_w, false);
    red[tid] = acc_k;
    __syncthreads();
    if (tid < D) {
        double s = 0.0;
        for (int l = 0; l < KL; ++l) s += red[l * D + tid];
        kbar[tid] = s / omega;
    }
    __syncthreads();
    red[tid] = acc_v;
    __syncthreads();
    if (tid < D) {
        double s = 0.0;
        for (int l = 0; l < KL; ++l) s += red[l * D + tid];
        vbar[tid] = s / omega;
    }
    __syncthreads();

    // pass 2: sum_j w_j (rho . (k_j - kbar)) (v_j - vbar)
    double acc_o = 0.0;
    for (int c0 = 0; c0 < cnt; c0 += G_CHK) {
        const int nk = min(G_CHK, cnt - c0);
        if (tid < nk) {
            const int j = c0 + tid;
            double tj = 0.0;
            for (int a = 0; a < D; ++a) tj += rs[a] * (load_f64(k + base, static_cast<int64_t>(j) * D + a) - kbar[a]);
            ws[tid] = exp(score(j) - m) * tj;
        }
        __syncthreads();
        for (int jj = kl; jj < nk; jj += KL)
            acc_o += ws[jj] * (load_f64(v + base, static_cast<int64_t>(c0 + jj) * D + fa) - vbar[fa]);
        __syncthreads();
    }
    red[tid] = acc_o;
    __syncthreads();
    if (tid < D) {
        double s = 0.0;
        for (int l = 0; l < KL; ++l) s += red[l * D + tid];
        out[base + static_cast<int64_t>(i) * D + tid] = static_cast<float>(vbar[tid] - s / omega);
    }
    if (stats != nullptr && tid == 0)   // the row's log-sum-exp of the scores, base 2
        stats[static_cast<int64_t>(bh) * n + i] = static_cast<float>((m + log(omega)) * 1.4426950408889634);
    __syncthreads();   // the shared arrays are free for the block's next row
}

template <typename TIn, int D>
__global__ __launch_bounds__(G_NT) void lla_parallax_exact_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v, const TIn* __restrict__ rho,
    float* __restrict__ out, float* __restrict__ stats, int n, int BH, double inv_h) {
    const int i = n - 1 - static_cast<int>(blockIdx.x / BH);   // longest rows first
    const int bh = static_cast<int>(blockIdx.x % BH);
    parallax_exact_row<TIn, D>(q, k, v, rho, out, stats, n, inv_h, i, bh);
}

// The rows of the heads the matrix-core kernel listed (range guard), by the same fp64 row
// code: a fixed grid strides over (listed head, row) pairs, longest rows first; with no head
// listed every block exits at once.
constexpr int G_FALLBACK_BLOCKS = 512;
__global__ __launch_bounds__(G_NT) void lla_parallax_fallback_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ rho, float* __restrict__ out, float* __restrict__ stats,
    const unsigned* __restrict__ nlisted, const int* __restrict__ hlist, int n, double inv_h) {
    const unsigned nh = *nlisted;
    const int64_t items = static_cast<int64_t>(nh) * n;
    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int bh = hlist[it % nh];
        const int i = n - 1 - static_cast<int>(it / nh);
        parallax_exact_row<uint16_t, FD>(q, k, v, rho, out, stats, n, inv_h, i, bh);
    }
}

template <typename TIn, int D>
hipError_t launch_parallax_exact_t(const Problem& p) {
    const int BH = static_cast<int>(p.B * p.H);
    const unsigned blocks = static_cast<unsigned>(p.B * p.H * p.n);
    prof_begin(p.stream, "lla_parallax_exact_kernel");
    lla_parallax_exact_kernel<TIn, D><<<dim3(blocks), dim3(G_NT), 0, p.stream>>>(
        static_cast<const TIn*>(p.q), static_cast<const TIn*>(p.k), static_cast<const TIn*>(p.v),
        static_cast<const TIn*>(p.rho), p.out, p.stats, static_cast<int>(p.n), BH, 1.0 / p.h);
    prof_end(p.stream);
    return hipGetLastError();
}

template <typename TIn>
hipError_t launch_parallax_exact_d(const Problem& p) {
    switch (p.d) {
        case 16: return launch_parallax_exact_t<TIn, 16>(p);
        case 32: return launch_parallax_exact_t<TIn, 32>(p);
        case 64: return launch_parallax_exact_t<TIn, 64>(p);
        case 128: return launch_parallax_exact_t<TIn, 128>(p);
        default: return hipErrorInvalidValue;
    }
}

// Workspace: tile images [B*H][tiles][X_TILE] | tile key sums [B*H][tiles][d] floats |
// tile max key norms [B*H][tiles] floats | tile max |v| [B*H][tiles] floats | count of
// listed heads (one unsigned) | listed heads [B*H] ints, regions 256-byte aligned.
struct ParallaxLayout {
    int64_t img, ksum, kmax, vmax, nlisted, hlist, total;
};

ParallaxLayout parallax_layout(int64_t BH, int64_t n) {
    auto up = [](int64_t bytes) { return (bytes + 255) & ~int64_t(255); };
    const int64_t tiles = (n + MT - 1) / MT;
    ParallaxLayout L;
    L.img = 0;
    L.ksum = L.img + up(BH * tiles * X_TILE);
    L.kmax = L.ksum + up(BH * tiles * FD * 4);
    L.vmax = L.kmax + up(BH * tiles * 4);
    L.nlisted = L.vmax + up(BH * tiles * 4);
    L.hlist = L.nlisted + up(4);
    L.total = L.hlist + up(BH * 4);
    return L;
}

}  // namespace

bool parallax_fast_supports(int dtype, int64_t d, int64_t n) {
    // Buffer resources address a head's tile images with 32-bit byte offsets.
    return dtype == 1 && d == FD && n <= kFastMaxN;
}

size_t parallax_workspace_bytes(int64_t B, int64_t H, int64_t n, int64_t d) {
    (void)d;
    return static_cast<size_t>(parallax_layout(B * H, n).total);
}

hipError_t launch_parallax_fast(const Problem& p, void* workspace) {
    const int n = static_cast<int>(p.n);
    const int BH = static_cast<int>(p.B * p.H);
    const int ptiles = (n + MT - 1) / MT;
    const ParallaxLayout L = parallax_layout(BH, n);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    unsigned char* img = ws + L.img;
    float* ksum = reinterpret_cast<float*>(ws + L.ksum);
    float* kmax = reinterpret_cast<float*>(ws + L.kmax);
    float* vmax = reinterpret_cast<float*>(ws + L.vmax);
    unsigned* nlisted = reinterpret_cast<unsigned*>(ws + L.nlisted);
    int* hlist = reinterpret_cast<int*>(ws + L.hlist);
    const auto* k = static_cast<const uint16_t*>(p.k);
    const auto* v = static_cast<const uint16_t*>(p.v);
    prof_begin(p.stream, "lla_parallax_pack_kernel");
    lla_parallax_pack_kernel<<<dim3(static_cast<unsigned>(BH) * ptiles), dim3(256), 0, p.stream>>>(
        k, v, img, ksum, kmax, vmax, nlisted, n, ptiles);
    prof_end(p.stream);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const unsigned blocks = static_cast<unsigned>(BH) * ((n + X_QB - 1) / X_QB);
    prof_begin(p.stream, "lla_parallax_kernel");
    if (p.stats != nullptr)
        lla_parallax_kernel<true><<<dim3(blocks), dim3(X_WAVES * 64), 0, p.stream>>>(
            static_cast<const uint16_t*>(p.q), static_cast<const uint16_t*>(p.rho), img, ksum, kmax, vmax, nlisted,
            hlist, p.out, p.stats, n, BH, static_cast<float>(LOG2E / p.h));
    else
        lla_parallax_kernel<false><<<dim3(blocks), dim3(X_WAVES * 64), 0, p.stream>>>(
            static_cast<const uint16_t*>(p.q), static_cast<const uint16_t*>(p.rho), img, ksum, kmax, vmax, nlisted,
            hlist, p.out, nullptr, n, BH, static_cast<float>(LOG2E / p.h));
    prof_end(p.stream);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t rows_all = static_cast<int64_t>(BH) * n;
    const unsigned fb = static_cast<unsigned>(rows_all < G_FALLBACK_BLOCKS ? rows_all : G_FALLBACK_BLOCKS);
    prof_begin(p.stream, "lla_parallax_fallback_kernel");
    lla_parallax_fallback_kernel<<<dim3(fb), dim3(G_NT), 0, p.stream>>>(
        static_cast<const uint16_t*>(p.q), static_cast<const uint16_t*>(p.k), static_cast<const uint16_t*>(p.v),
        static_cast<const uint16_t*>(p.rho), p.out, p.stats, nlisted, hlist, n, 1.0 / p.h);
    prof_end(p.stream);
    return hipGetLastError();
}

hipError_t launch_parallax_exact(const Problem& p) {
    return p.dtype == 0 ? launch_parallax_exact_d<float>(p) : launch_parallax_exact_d<uint16_t>(p);
}

}  // namespace lla
