// Device-side helpers shared by the matrix-core kernels of liblla (gfx950): operand
// vector types, MFMA wrappers, wave-uniform pointers and the XCD-aware block order.
//
// MFMA: v_mfma_f32_16x16x32_{bf16,f16}.  Lane l supplies row/column (l % 16) of A/B and 8
// consecutive K-slots (l / 16); D[4 (l/16) + r][l % 16] lands in accumulator register r.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lla {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int FD = 64;              // head dimension of the matrix-core kernels
constexpr float LOG2E = 1.4426950408889634f;

// Reproduction check of the matrix-core paths: NCHK projections of the centred keys on fixed
// +-1 directions (Walsh functions), 5 KiB per 64-key tile for their fp16 image and the
// per-key |v - a_v|^2; rows whose estimated relative error exceeds CHK_TOL go to the fp64
// kernel.
constexpr int NCHK = 32;
constexpr int KU_TILE_BYTES = 5 * 1024;
// Column of key jt (0..63 within a 64-key tile) in the feature-major value images and check
// images the probe passes read: within each 32-key group, key 16h + 4g + r sits at
// 8g + 4h + r, so that the 8 keys MFMA K-slot g takes from the probe weights (keys 4g..
// and 16 + 4g.. of the score layout) are one 16-byte read.
__host__ __device__ constexpr int vcol(int jt) {
    return (jt & ~31) | (((jt >> 2) & 3) << 3) | (((jt >> 4) & 1) << 2) | (jt & 3);
}
constexpr float CHK_TOL = 1.5e-3f;

// Compiler fence for wave-private LDS exchanges: a lane reads words that other lanes of
// the same wave stored, so no LDS access may move across a publish/consume boundary.
// (A blocked variant of the LLA solve was miscompiled without such fences on gfx950:
// an LDS access moved across a dependent one.  The fences cost no instructions.)
#define LDS_FENCE() __asm__ volatile("" ::: "memory")

// A wave-uniform pointer, rebuilt from scalar registers so that memory instructions can use
// the scalar-base addressing form.
__device__ __forceinline__ const unsigned char* uniform_ptr(const unsigned char* p) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
    return reinterpret_cast<const unsigned char*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Value of x in lane `src` (a compile-time lane), broadcast to the wave.
__device__ __forceinline__ float lane_value(float x, int src) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), src));
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Element idx of an fp32 or bf16 (raw bits) array, exactly, as fp64.
__device__ __forceinline__ double load_f64(const float* p, int64_t idx) { return static_cast<double>(p[idx]); }
__device__ __forceinline__ double load_f64(const uint16_t* p, int64_t idx) {
    return static_cast<double>(__uint_as_float(static_cast<uint32_t>(p[idx]) << 16));
}

__device__ __forceinline__ float4v mfma_bf16(bf16x8 a, bf16x8 b, float4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float4v mfma_f16(half8 a, half8 b, float4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Guard of the matrix-core paths' fp16 images.  `guard` (workspace, unsigned words): [0] the
// number of rows handed back to the fp64 kernel, [1 + 2 bh] and [2 + 2 bh] the largest
// |k - a| and |v - a_v| of head bh (fp32 bit patterns of non-negative values, so the integer
// maximum is the float maximum); `list` (workspace): the handed-back rows, entries bh * n + i.
// A head whose centred keys or values leave the range where their fp16 images are accurate
// (above 2^14, near the fp16 maximum 65504; or non-zero but below 2^-10, where the fp16
// spacing is no longer small against them) has every row of the path recomputed in fp64; so
// has every row whose output is not finite, or whose solve dropped a pivot although the ridge
// keeps its system positive definite.
__device__ __forceinline__ bool head_unsafe(const unsigned* guard, int bh) {
    // Maxima are stored as the bits of non-negative floats, so unsigned order is float
    // order (and a NaN or inf reads as too large).  Safe range: 2^-10 <= max <= 2^14.
    const unsigned mk = guard[1 + 2 * bh], mv = guard[2 + 2 * bh];
    const unsigned hi = 0x46800000u, lo = 0x3A800000u;
    return mk > hi || mv > hi || (mk != 0u && mk < lo) || (mv != 0u && mv < lo);
}
__device__ __forceinline__ void hand_back(unsigned* guard, int* list, int bh, int n, int i) {
    const unsigned slot = atomicAdd(guard, 1u);
    list[slot] = bh * n + i;
}
// Largest x >= 0 over the wave (in every lane).
__device__ __forceinline__ float wave_max_nonneg(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

// In-place Walsh-Hadamard transform of N values in registers (N a power of two):
// x[m] <- sum_f (-1)^popcount(f & m) x[f].
template <int N>
__device__ __forceinline__ void walsh_transform(float (&x)[N]) {
#pragma unroll
    for (int hh = 1; hh < N; hh <<= 1)
#pragma unroll
        for (int i = 0; i < N; i += 2 * hh)
#pragma unroll
            for (int e = i; e < i + hh; ++e) {
                const float a0 = x[e], a1 = x[e + hh];
                x[e] = a0 + a1;
                x[e + hh] = a0 - a1;
            }
}

// Block b -> (head bh, row block blk).  Work-groups go round-robin to the 8 XCDs, so
// b % 8 picks the XCD: heads are taken 8 at a time (head 8 G + b % 8 on XCD b % 8) and, in
// each group of 8, row blocks run longest first.  Each XCD's L2 then holds the packed K/V of
// about one head at a time instead of a quarter of all heads.
__device__ __forceinline__ void head_major_block(int b, int BH, int nblk, int* bh, int* blk) {
    const int full = BH / 8, span = 8 * nblk;
    int hg, r, hcnt;
    if (b < full * span) {
        hg = b / span; r = b - hg * span; hcnt = 8;
    } else {
        hg = full; r = b - full * span; hcnt = BH - 8 * full;
    }
    *blk = nblk - 1 - r / hcnt;
    *bh = 8 * hg + r % hcnt;
}

}  // namespace
}  // namespace lla
