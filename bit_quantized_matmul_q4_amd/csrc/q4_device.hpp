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
// The order (version 1), for output (m, n), K = 32 * nb:
//   quads:    G = ceil(nb / 4) groups of 4 blocks; the last may be short.
//   segments: S = min(16, 2^floor(log2 G)); segment j covers quads
//             [floor(j G / S), floor((j+1) G / S)), i.e. blocks
//             [4 floor(j G / S), min(nb, 4 floor((j+1) G / S))).
//   block dot: s_b = element (m, n) of ONE v_mfma_f32_16x16x32_{bf16,f16}
//             with C = 0, A row = x[m][32b .. 32b+31] in natural k order,
//             B column = (q[n][32b+k] - 8) / 16, exact in x's 16-bit type.
//   segment:  p_j = +0; for b ascending: p_j = fmaf(d[n][b], s_b, p_j).
//   tree:     for h = 1, 2, 4, .. S/2: p_j = p_j + p_{j+h} for j % 2h == 0.
//   output:   y[m][n] = 16 * p_0   (exact: undoes the 1/16 of the operand).
// S depends on K only, so slicing N (sharding) keeps every bit.
//
// Weight layout read by the kernels (written by q4_pack): tiles of 16
// columns (t = n / 16, c = n % 16) by one quad (q = b / 4, i = b % 4),
// ordered [ceil(N/16)][G].  A tile holds 1024 code bytes, 16 per lane of a
// wave in lane order l = 16 g + c: bytes 4 i .. 4 i + 3 of lane l are bytes
// 4 g .. 4 g + 3 of block 4 q + i of column n in the row-major packing
// (codes of k = 32 b + 8 g .. + 7, low nibble first).  So one 16-byte load
// gives lane (g, c) exactly the B-operand dwords of the tile's four block
// dots.  Then 64 fp16 scales, [c][i].  Padding (n >= N, b >= nb) is zero.
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
// v_cvt_off_f32_i4 reads bits 3..0 of its source as a signed 4-bit integer
// t and returns t / 16.  With t = q ^ 8, t is q - 8 in two's complement, so
// each call yields (q - 8) / 16 exactly.  Only the compiler builtin is used
// (no inline assembly): the compiler then tracks every register the
// conversions write against in-flight matrix-core instructions.
__device__ __forceinline__ float i4_at(uint32_t v) { return __builtin_amdgcn_cvt_off_f32_i4((int)v); }

template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi)
{
    if constexpr (BF16) {
        const bf16x2 v = {(__bf16)lo, (__bf16)hi};  // v_cvt_pk_bf16_f32; exact here
        return __builtin_bit_cast(uint32_t, v);
    } else {
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));  // exact here
    }
}

// Eight codes (one packed dword: code of k = i in bits 4i..4i+3) -> the
// eight operand values (q - 8)/16 in natural k order, two per dword.
template <bool BF16>
__device__ __forceinline__ u32x4 dequant8(uint32_t w)
{
    const uint32_t t = w ^ 0x88888888u;
    const uint32_t h = (w >> 4) ^ 0x08888888u;
    u32x4 r;
    r.x = pack2<BF16>(i4_at(t), i4_at(h));
    r.y = pack2<BF16>(i4_at(t >> 8), i4_at(h >> 8));
    r.z = pack2<BF16>(i4_at(t >> 16), i4_at(h >> 16));
    r.w = pack2<BF16>(i4_at(t >> 24), i4_at(h >> 24));
    return r;
}

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

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// p = fmaf(d, s, p) for the four accumulator rows a lane holds.
__device__ __forceinline__ void scale_accumulate(f32x4 &p, float d, f32x4 s)
{
    p.x = __builtin_fmaf(d, s.x, p.x);
    p.y = __builtin_fmaf(d, s.y, p.y);
    p.z = __builtin_fmaf(d, s.z, p.z);
    p.w = __builtin_fmaf(d, s.w, p.w);
}

// Streaming form of the pairwise tree for one wave that owns an aligned run
// of L segments (L a power of two, at most 2^LV): call after each finished
// segment li = 0..L-1 with its partial in cur.  Left subtrees wait in stack
// (a binary counter over li); after li = L-1, cur holds the run's subtree
// root and the call returns true.  Otherwise cur must restart from +0.
template <int LV, int NACC>
__device__ __forceinline__ bool tree_push(f32x4 (&stack)[LV][NACC], f32x4 (&cur)[NACC], int li, int L)
{
    int lvl = 0;
#pragma unroll
    for (int l = 0; l < LV; ++l) {
        if (lvl == l && ((li >> l) & 1)) {
#pragma unroll
            for (int a = 0; a < NACC; ++a)
                cur[a] = stack[l][a] + cur[a];
            lvl = l + 1;
        }
    }
    if ((1 << lvl) >= L)
        return true;
#pragma unroll
    for (int l = 0; l < LV; ++l)
        if (l == lvl)
#pragma unroll
            for (int a = 0; a < NACC; ++a)
                stack[l][a] = cur[a];
    return false;
}

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
