// q4_device.hpp -- device primitives shared by both Q4 kernels (gfx950).
//
// Both kernels compute every output through the same fixed reduction order,
// so a row's bits do not depend on M, on the row's position in the batch, on
// the other rows, or on which kernel ran.  That property answers the failure
// traced in "Why Continuous Batching Slowed Down My LLM Inference Engine: A
// Metal Kernel Investigation" (sections "Same Prompt, Different Story" and
// "The Other Request Already Finished"): the matrix-vector and matrix-matrix
// kernels summed in different orders and dequantized at different times, so
// a batching decision changed the numbers written to the KV cache.
//
// The order (version 4), for output (m, n), K = 32 * nb:
//   quads:    G = ceil(nb / 4) groups of 4 blocks; the last may be short.
//   segments: S = min(16, 2^floor(log2 G)); segment j covers quads
//             [floor(j G / S), floor((j+1) G / S)), i.e. blocks
//             [4 floor(j G / S), min(nb, 4 floor((j+1) G / S))).
//   block dot s_b, v_mfma_f32_16x16x32_{bf16,f16} with A row =
//             x[m][32b .. 32b+31] in natural k order:
//             fp16 x: s_b = MFMA(A, B, C = 0), B column = q[n][32b+k] - 8
//               (exact in fp16), so every product is exact and a zero
//               weight adds exactly 0;
//             bf16 x: the correction C_b = MFMA(A, -24, C = 0) (every B
//               entry -24; depends on x only), then s_b = MFMA(A, B, C =
//               C_b) with B column = 16 + q[n][32b+k] (both operands exact
//               in bf16): the matrix core adds the correction to the sum of
//               the products itself.  A block of all-8 codes gives s_b = 0
//               exactly.  (bf16 has no packed add on this target, so an
//               exact q - 8 operand would cost about three times the
//               dequantization work; the offset 16 keeps the cancellation
//               to a factor 24 of the weight step.)
//   segment:  p_j = +0; for b ascending: p_j = fmaf(d[n][b], s_b, p_j).
//   tree:     for h = 1, 2, 4, .. S/2: p_j = p_j + p_{j+h} for j % 2h == 0.
//   output:   y[m][n] = p_0.
// S depends on K only, so slicing N (sharding) keeps every bit.
//
// Weight layout read by the kernels (written by q4_pack): tiles of 16
// columns (t = n / 16, c = n % 16) by one quad (q = b / 4, i = b % 4),
// ordered [ceil(N/16)][G].  A tile holds 1024 code bytes, 16 per lane of a
// wave in lane order l = 16 g + c: the little-endian word at bytes 4 i ..
// 4 i + 3 of lane l holds the codes of column n, k = 32 b + 8 g + r,
// r = 0..7, with code r at bit 4 (r / 2) + 16 (r % 2).  So one 16-byte load
// gives lane (g, c) its B-operand codes of the tile's four block dots, and
// a shift and a mask-and-or per pair of k turn them into operand words.
// Then 64 fp16 scales, [c][i].  Padding (n >= N, b >= nb) is zero.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4_plan.hpp"

namespace q4 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- dequant
// bf16: the 16-bit pattern 0x4180 | (q << 3), q in 0..15, is 16 + q exactly
// (16 = 0x4180, the code in the top four of the seven mantissa bits).
// fp16: 0x6400 | q is 1024 + q exactly (the ulp on [1024, 2048) is 1) and
// 0x6400 | (q << 4) is 1024 + 16 q; one packed fp16 add of -1032, or one
// packed fma by 1/16 with -72, leaves q - 8 (exact: the result is an integer
// in -8..7).  So the codes at bits 4..7 of each half need no shift.
template <bool BF16>
constexpr uint32_t kMask = BF16 ? 0x00780078u : 0x000F000Fu;
template <bool BF16>
constexpr uint32_t kMagic = BF16 ? 0x41804180u : 0x64006400u;
constexpr uint32_t kF16MaskHi = 0x00F000F0u;   // codes at bits 4..7 of each half
constexpr uint32_t kF16Bias = 0xE408E408u;     // -1032, -1032 (binary16)
constexpr uint32_t kF16Sixteenth = 0x2C002C00u;  // 1/16, 1/16
constexpr uint32_t kF16Bias16 = 0xD480D480u;   // -72, -72
// B operand of the bf16 correction dot: -24 in every entry.
constexpr uint32_t kBf16Offset = 0xC1C0C1C0u;
// Whether the block dot carries the correction (bf16) or is exact (fp16).
template <bool BF16>
constexpr bool kCorrected = BF16;

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// The dequant constants in registers the compiler cannot fold: the masks and
// the fp16 biases in scalar registers, the magic and 1/16 in vector ones (one
// scalar operand per instruction on this target; three-operand instructions
// take no literal).  The empty statements emit no instructions.  The bf16
// correction's B operand (-24 everywhere) is built once the same way, so the
// compiler keeps it in four registers instead of rebuilding it for every
// block dot.
template <bool BF16>
struct Dequant {
    uint32_t mask, magic, mask_hi, bias, bias16, sixteenth;
    u32x4 offset;
    __device__ __forceinline__ Dequant()
    {
        mask = kMask<BF16>;
        magic = kMagic<BF16>;
        asm volatile("" : "+s"(mask));
        asm volatile("" : "+v"(magic));
        if constexpr (BF16) {
            mask_hi = bias = bias16 = sixteenth = 0u;
            offset = (u32x4){kBf16Offset, kBf16Offset, kBf16Offset, kBf16Offset};
            asm volatile("" : "+v"(offset));
        } else {
            mask_hi = kF16MaskHi;
            bias = kF16Bias;
            bias16 = kF16Bias16;
            sixteenth = kF16Sixteenth;
            offset = (u32x4){0u, 0u, 0u, 0u};
            asm volatile("" : "+s"(mask_hi));
            asm volatile("" : "+s"(bias));
            asm volatile("" : "+s"(bias16));
            asm volatile("" : "+v"(sixteenth));
        }
    }

    // One packed word (code r at bit 4 (r / 2) + 16 (r % 2)) -> the eight
    // operand values in natural k order, two per dword.  bf16: each pair's
    // codes moved to bits 3..6 of each half (pair 0 up by 3, pairs 1..3 down
    // by 1, 5, 9), masked and or-ed with the magic: 8 operations.  fp16:
    // pairs 0 and 1 masked in place, pairs 2 and 3 from one shift by 8, then
    // the packed add (pairs 0, 2) or fma (pairs 1, 3): 9 operations.
    __device__ __forceinline__ u32x4 operator()(uint32_t w) const
    {
        u32x4 r;
        if constexpr (BF16) {
            r.x = ((w << 3) & mask) | magic;
            r.y = ((w >> 1) & mask) | magic;
            r.z = ((w >> 5) & mask) | magic;
            r.w = ((w >> 9) & mask) | magic;
        } else {
            const f16x2 b = __builtin_bit_cast(f16x2, bias);
            const f16x2 b16 = __builtin_bit_cast(f16x2, bias16);
            const f16x2 s16 = __builtin_bit_cast(f16x2, sixteenth);
            const uint32_t w8 = w >> 8;
            const f16x2 v0 = __builtin_bit_cast(f16x2, (w & mask) | magic);
            const f16x2 v1 = __builtin_bit_cast(f16x2, (w & mask_hi) | magic);
            const f16x2 v2 = __builtin_bit_cast(f16x2, (w8 & mask) | magic);
            const f16x2 v3 = __builtin_bit_cast(f16x2, (w8 & mask_hi) | magic);
            r.x = __builtin_bit_cast(uint32_t, v0 + b);
            r.y = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(v1, s16, b16));
            r.z = __builtin_bit_cast(uint32_t, v2 + b);
            r.w = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(v3, s16, b16));
        }
        return r;
    }
};

// ---------------------------------------------------------------- BlockDot
// One v_mfma_f32_16x16x32 with C = 0.  Lane l supplies A[l % 16][8 (l/16) ..
// 8 (l/16) + 7] and B[8 (l/16) .. +7][l % 16] (eight 16-bit values in four
// dwords) and receives D[4 (l/16) + i][l % 16] for i = 0..3.
template <bool BF16>
__device__ __forceinline__ f32x4 blockdot(u32x4 a, u32x4 b)
{
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), zero, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), zero, 0, 0, 0);
}

// The same with the accumulator input C.
template <bool BF16>
__device__ __forceinline__ f32x4 blockdot_acc(u32x4 a, u32x4 b, f32x4 c)
{
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// The block's correction C_b = MFMA(A, -24) (bf16; x only), or zero (fp16:
// unused).
template <bool BF16>
__device__ __forceinline__ f32x4 correction(u32x4 a, const Dequant<BF16> &dq)
{
    if constexpr (kCorrected<BF16>)
        return blockdot<BF16>(a, dq.offset);
    else
        return (f32x4){0.f, 0.f, 0.f, 0.f};
}

// The block dot s_b with the operand b dequantized: MFMA(A, b, C = C_b)
// (bf16) or MFMA(A, b, C = 0) (fp16).
template <bool BF16>
__device__ __forceinline__ f32x4 block_dot(u32x4 a, u32x4 b, f32x4 cb)
{
    if constexpr (kCorrected<BF16>)
        return blockdot_acc<BF16>(a, b, cb);
    else
        return blockdot<BF16>(a, b);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// p = fmaf(d, s_b, p) for the four accumulator rows a lane holds.
__device__ __forceinline__ void scale_accumulate(f32x4 &p, float d, f32x4 s)
{
    p.x = __builtin_fmaf(d, s.x, p.x);
    p.y = __builtin_fmaf(d, s.y, p.y);
    p.z = __builtin_fmaf(d, s.z, p.z);
    p.w = __builtin_fmaf(d, s.w, p.w);
}

// Streaming form of the pairwise tree for one wave that owns an aligned run
// of L <= 16 segments (L a power of two): push() after each finished
// segment li = 0..L-1 with its partial in cur.  Left subtrees wait at the
// levels: the trailing one-bits of li name the levels that merge into cur
// (left operand first), the first zero-bit the level cur then waits at.
// After li = L-1, cur holds the run's subtree root and push() returns true;
// otherwise cur must restart from +0.  The levels are separate named
// registers written by value (selects or uniform branches), never through
// an index or a pointer, so they cannot fall back to scratch memory.
template <int NACC, typename T>
struct TreeStack {
    T s0[NACC], s1[NACC], s2[NACC], s3[NACC];

    // Per-element selects over every level: no branches (the form for
    // frequent pushes of few values).
    __device__ __forceinline__ bool push(T (&cur)[NACC], int li, int L)
    {
        const bool m0 = li & 1, m1 = m0 && (li & 2), m2 = m1 && (li & 4), m3 = m2 && (li & 8);
#pragma unroll
        for (int a = 0; a < NACC; ++a) {
            if (m0)
                cur[a] = s0[a] + cur[a];
            if (m1)
                cur[a] = s1[a] + cur[a];
            if (m2)
                cur[a] = s2[a] + cur[a];
            if (m3)
                cur[a] = s3[a] + cur[a];
        }
        const bool root = li == L - 1;
        const bool w0 = !root && !m0, w1 = !root && m0 && !m1, w2 = !root && m1 && !m2, w3 = !root && m2 && !m3;
#pragma unroll
        for (int a = 0; a < NACC; ++a) {
            s0[a] = w0 ? cur[a] : s0[a];
            s1[a] = w1 ? cur[a] : s1[a];
            s2[a] = w2 ? cur[a] : s2[a];
            s3[a] = w3 ? cur[a] : s3[a];
        }
        return root;
    }

    // Same result with real scalar branches: only the merging levels are
    // added and one level is written (the form for many values per push).
    __device__ __forceinline__ bool push_branch(T (&cur)[NACC], int li, int L)
    {
        // li is wave-uniform.  The empty volatile statements keep the
        // compiler from turning the branches back into selects.
        const int t = __builtin_amdgcn_readfirstlane(__builtin_ctz(~li));  // trailing one-bits
        if (t > 0) {
            asm volatile("");
#pragma unroll
            for (int a = 0; a < NACC; ++a)
                cur[a] = s0[a] + cur[a];
        }
        if (t > 1) {
            asm volatile("");
#pragma unroll
            for (int a = 0; a < NACC; ++a)
                cur[a] = s1[a] + cur[a];
        }
        if (t > 2) {
            asm volatile("");
#pragma unroll
            for (int a = 0; a < NACC; ++a)
                cur[a] = s2[a] + cur[a];
        }
        if (t > 3) {
            asm volatile("");
#pragma unroll
            for (int a = 0; a < NACC; ++a)
                cur[a] = s3[a] + cur[a];
        }
        const bool root = li == L - 1;
        if (!root) {
            asm volatile("");
            if (t == 0) {
                asm volatile("");
#pragma unroll
                for (int a = 0; a < NACC; ++a)
                    s0[a] = cur[a];
            } else if (t == 1) {
                asm volatile("");
#pragma unroll
                for (int a = 0; a < NACC; ++a)
                    s1[a] = cur[a];
            } else if (t == 2) {
                asm volatile("");
#pragma unroll
                for (int a = 0; a < NACC; ++a)
                    s2[a] = cur[a];
            } else {
                asm volatile("");
#pragma unroll
                for (int a = 0; a < NACC; ++a)
                    s3[a] = cur[a];
            }
        }
        return root;
    }
};

// Pairwise tree over v[0..S): the fixed order of the contract.
template <int SMAX>
__device__ __forceinline__ float tree_sum(float (&v)[SMAX], int S)
{
#pragma unroll
    for (int h = 1; h < SMAX; h *= 2) {
#pragma unroll
        for (int j = 0; j + h < SMAX; j += 2 * h)
            if (j + h < S)
                v[j] = v[j] + v[j + h];
    }
    return v[0];
}

}  // namespace q4
