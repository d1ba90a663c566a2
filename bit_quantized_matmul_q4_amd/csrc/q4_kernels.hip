// q4_kernels.hip -- the Q4 linear kernels for gfx950 (MI355X).
//
// Two kernels compute y = x . dequant(Wq)^T, as the matrix-vector and
// matrix-matrix kernels of "Why Continuous Batching Slowed Down My LLM
// Inference Engine: A Metal Kernel Investigation" (section "Two Rows of
// Input, Two Different Kernels") do, but through one fixed reduction order
// (q4_device.hpp), so they return identical bits:
//
//  * q4_gemv: the weight-streaming kernel for small M.  One workgroup owns 16
//    output columns; its S waves each own one K-segment, stream that
//    segment's packed codes and scales from HBM once, dequantize in
//    registers while reading (the matrix-vector kernel's advantage the page
//    names), and run the block dots on MFMA with all (<= 16) rows of x in
//    the A operand.  The S segment partials meet in LDS for the pairwise
//    tree.  Rows beyond 16 run as further 16-row slices (grid.y).
//
//  * q4_gemm: the LDS-staged tile kernel for larger M.  A workgroup owns a
//    64 x 64 output tile; per group of four blocks it dequantizes the 64 x
//    128 weight tile into LDS once and stages the 64 x 128 activation tile,
//    and four waves run 2 x 2 MFMA tiles each from LDS.  K may be split
//    across workgroups (one subtree of segments each) when a workspace is
//    given; q4_tree_combine then joins the subtree roots in tree order.
//
//  * q4_pack_kernel: nibble packing of 4-bit codes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4_device.hpp"
#include "q4_launch.hpp"

namespace q4 {

// =================================================================== GEMV
// grid = (ceil(N/16), ceil(M/16)), block = 64 * S threads (wave j = segment j).
template <bool BF16>
__global__ __launch_bounds__(1024) void q4_gemv(const uint16_t *__restrict__ x,
                                                const uint8_t *__restrict__ wq,
                                                const uint16_t *__restrict__ scales,
                                                float *__restrict__ y, int M, int N, int K, Plan plan)
{
    __shared__ float red[16][16][17];  // [segment][row slot][column slot], padded

    const int lane = threadIdx.x & 63;
    const int seg = threadIdx.x >> 6;
    const int g = lane >> 4;   // lane group: k-slots 8g..8g+7, output rows 4g..4g+3
    const int c = lane & 15;   // column slot (B, D) and row slot (A)
    const int n = blockIdx.x * 16 + c;
    const int m0 = blockIdx.y * 16;
    const int mrows = min(16, M - m0);
    const bool col_ok = n < N;
    const bool row_ok = c < mrows;

    const size_t half_k = (size_t)K / 2;
    const size_t nblk_row = (size_t)K / 32;
    const uint8_t *wrow = wq + (size_t)(col_ok ? n : 0) * half_k + 4 * g;
    const uint16_t *srow = scales + (size_t)(col_ok ? n : 0) * nblk_row;
    const uint16_t *xrow = x + (size_t)(m0 + (row_ok ? c : 0)) * K + 8 * g;

    const int b_begin = seg_first_block(plan, seg);
    const int b_end = seg_end_block(plan, seg);

    f32x4 p = {0.f, 0.f, 0.f, 0.f};
    for (int b0 = b_begin; b0 < b_end; b0 += 4) {
        const int nq = min(4, b_end - b0);
        uint32_t w[4];
        uint32_t d[4];
        u32x4 xa[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = i < nq;
            w[i] = (ok && col_ok) ? *(const uint32_t *)(wrow + (size_t)(b0 + i) * 16) : 0x88888888u;
            d[i] = (ok && col_ok) ? srow[b0 + i] : 0u;
            xa[i] = (ok && row_ok) ? *(const u32x4 *)(xrow + (size_t)(b0 + i) * 32) : (u32x4){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i < nq) {
                const f32x4 s = blockdot<BF16>(xa[i], dequant8<BF16>(w[i]));
                scale_accumulate(p, half_bits_to_float(d[i]), s);
            }
        }
    }

    red[seg][4 * g + 0][c] = p.x;
    red[seg][4 * g + 1][c] = p.y;
    red[seg][4 * g + 2][c] = p.z;
    red[seg][4 * g + 3][c] = p.w;
    __syncthreads();

    if (seg == 0) {
        const int S = plan.S;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float v[16];
#pragma unroll
            for (int j = 0; j < 16; ++j)
                v[j] = j < S ? red[j][4 * g + r][c] : 0.f;
            const float root = tree_sum<16>(v, S);
            const int row = 4 * g + r;
            if (row < mrows && col_ok)
                y[(size_t)(m0 + row) * N + n] = root * 16.0f;
        }
    }
}

// =================================================================== GEMM
constexpr int GEMM_BM = 64;
constexpr int GEMM_BN = 64;
constexpr int GEMM_LDK = 128 + 8;  // 16-bit elements per staged row (padded)

// grid = (ceil(N/64), ceil(M/64), Gk), block = 256.  K-group z owns the
// segments [z S/Gk, (z+1) S/Gk) -- a complete subtree of the pairwise tree.
template <bool BF16>
__global__ __launch_bounds__(256) void q4_gemm(const uint16_t *__restrict__ x,
                                               const uint8_t *__restrict__ wq,
                                               const uint16_t *__restrict__ scales,
                                               float *__restrict__ out, int M, int N, int K,
                                               Plan plan, int Gk, int write_partial)
{
    __shared__ __attribute__((aligned(16))) uint16_t xs[GEMM_BM][GEMM_LDK];
    __shared__ __attribute__((aligned(16))) uint16_t ws[GEMM_BN][GEMM_LDK];
    __shared__ float ds[4][GEMM_BN];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    const int g = lane >> 4, c = lane & 15;
    const int n0 = blockIdx.x * GEMM_BN;
    const int m0 = blockIdx.y * GEMM_BM;
    const int z = blockIdx.z;

    const int L = plan.S / Gk;       // segments of this K-group (power of two)
    const int j0 = z * L;

    // staging roles: thread -> (tile row/column r, block-in-quad q)
    const int st_r = tid >> 2;
    const int st_q = tid & 3;
    const int st_n = n0 + st_r;
    const int st_m = m0 + st_r;
    const bool st_col_ok = st_n < N;
    const bool st_row_ok = st_m < M;
    const size_t half_k = (size_t)K / 2;
    const size_t nblk_row = (size_t)K / 32;

    f32x4 p[2][2];
    f32x4 stack[4][2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
            p[a][b] = (f32x4){0.f, 0.f, 0.f, 0.f};

    for (int li = 0; li < L; ++li) {
        const int seg = j0 + li;
        const int b_begin = seg_first_block(plan, seg);
        const int b_end = seg_end_block(plan, seg);
        for (int b0 = b_begin; b0 < b_end; b0 += 4) {
            const int nq = min(4, b_end - b0);
            // ---- stage: dequantized weights, activations, scales
            {
                const bool okb = st_q < nq;
                u32x4 wv = {0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
                uint32_t dv = 0u;
                if (okb && st_col_ok) {
                    wv = *(const u32x4 *)(wq + (size_t)st_n * half_k + (size_t)(b0 + st_q) * 16);
                    dv = scales[(size_t)st_n * nblk_row + b0 + st_q];
                }
                u32x4 *wdst = (u32x4 *)&ws[st_r][st_q * 32];
                wdst[0] = dequant8<BF16>(wv.x);
                wdst[1] = dequant8<BF16>(wv.y);
                wdst[2] = dequant8<BF16>(wv.z);
                wdst[3] = dequant8<BF16>(wv.w);
                ds[st_q][st_r] = half_bits_to_float(dv);

                u32x4 *xdst = (u32x4 *)&xs[st_r][st_q * 32];
                if (okb && st_row_ok) {
                    const u32x4 *xsrc = (const u32x4 *)(x + (size_t)st_m * K + (size_t)(b0 + st_q) * 32);
                    xdst[0] = xsrc[0];
                    xdst[1] = xsrc[1];
                    xdst[2] = xsrc[2];
                    xdst[3] = xsrc[3];
                } else {
                    const u32x4 zero = {0u, 0u, 0u, 0u};
                    xdst[0] = zero;
                    xdst[1] = zero;
                    xdst[2] = zero;
                    xdst[3] = zero;
                }
            }
            __syncthreads();
            // ---- compute: 2 x 2 MFMA tiles per wave per block
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i < nq) {
                    u32x4 a[2], b[2];
                    float dsc[2];
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        a[t] = *(const u32x4 *)&xs[32 * wr + 16 * t + c][i * 32 + 8 * g];
                        b[t] = *(const u32x4 *)&ws[32 * wc + 16 * t + c][i * 32 + 8 * g];
                        dsc[t] = ds[i][32 * wc + 16 * t + c];
                    }
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                        for (int ct = 0; ct < 2; ++ct)
                            scale_accumulate(p[rt][ct], dsc[ct], blockdot<BF16>(a[rt], b[ct]));
                }
            }
            __syncthreads();
        }
        // ---- segment done: merge into the pairwise tree (binary counter)
        f32x4 cur[2][2];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                cur[a][b] = p[a][b];
                p[a][b] = (f32x4){0.f, 0.f, 0.f, 0.f};
            }
        int lvl = 0;
#pragma unroll
        for (int l = 0; l < 4; ++l) {
            if (lvl == l && ((li >> l) & 1)) {
#pragma unroll
                for (int a = 0; a < 2; ++a)
#pragma unroll
                    for (int b = 0; b < 2; ++b)
                        cur[a][b] = stack[l][a][b] + cur[a][b];
                lvl = l + 1;
            }
        }
        // a left child waits on its level; the root (lvl == log2 L) stays in cur
        if ((1 << lvl) < L) {
#pragma unroll
            for (int l = 0; l < 4; ++l)
                if (l == lvl)
#pragma unroll
                    for (int a = 0; a < 2; ++a)
#pragma unroll
                        for (int b = 0; b < 2; ++b)
                            stack[l][a][b] = cur[a][b];
        } else {
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    p[a][b] = cur[a][b];  // keep the subtree root
        }
    }

    // ---- write: y = 16 * root, or the unscaled subtree root to the workspace
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const int n = n0 + 32 * wc + 16 * ct + c;
            if (n >= N)
                continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + 32 * wr + 16 * rt + 4 * g + r;
                if (m >= M)
                    continue;
                const float v = r == 0 ? p[rt][ct].x : r == 1 ? p[rt][ct].y : r == 2 ? p[rt][ct].z : p[rt][ct].w;
                if (write_partial)
                    out[((size_t)z * M + m) * N + n] = v;
                else
                    out[(size_t)m * N + n] = v * 16.0f;
            }
        }
}

// Joins Gk subtree roots (workspace [Gk][M][N]) in pairwise-tree order.
__global__ __launch_bounds__(256) void q4_tree_combine(const float *__restrict__ part,
                                                       float *__restrict__ y, size_t MN, int Gk)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= MN)
        return;
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
        v[j] = j < Gk ? part[(size_t)j * MN + i] : 0.f;
    y[i] = tree_sum<16>(v, Gk) * 16.0f;
}

// =================================================================== pack
// Output byte o of the flat [N][K/2] array takes codes 2o and 2o+1 of the
// flat [N][K] array; each thread writes 16 output bytes.
__global__ __launch_bounds__(256) void q4_pack_kernel(const uint8_t *__restrict__ codes,
                                                      uint8_t *__restrict__ wq, size_t chunks)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= chunks)
        return;
    const uint8_t *src = codes + 32 * i;
    uint32_t out[4];
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
        uint32_t v = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t lo = src[8 * wd + 2 * b] & 0x0Fu;
            const uint32_t hi = src[8 * wd + 2 * b + 1] & 0x0Fu;
            v |= (lo | (hi << 4)) << (8 * b);
        }
        out[wd] = v;
    }
    *(u32x4 *)(wq + 16 * i) = (u32x4){out[0], out[1], out[2], out[3]};
}

// ============================================================== launchers
hipError_t launch_gemv(const void *x, bool bf16, const uint8_t *wq, const uint16_t *scales,
                       float *y, int M, int N, int K, hipStream_t stream)
{
    const Plan plan = make_plan(K);
    const dim3 grid((N + 15) / 16, (M + 15) / 16);
    const dim3 block(64 * plan.S);
    if (bf16)
        hipLaunchKernelGGL(q4_gemv<true>, grid, block, 0, stream, (const uint16_t *)x, wq, scales, y,
                           M, N, K, plan);
    else
        hipLaunchKernelGGL(q4_gemv<false>, grid, block, 0, stream, (const uint16_t *)x, wq, scales, y,
                           M, N, K, plan);
    return hipGetLastError();
}

static int gemm_split(int M, int N, int K, size_t workspace_bytes)
{
    const Plan plan = make_plan(K);
    const long long tiles = (long long)((M + GEMM_BM - 1) / GEMM_BM) * ((N + GEMM_BN - 1) / GEMM_BN);
    int gk = 1;
    while (gk < plan.S && tiles * gk < 1024)
        gk *= 2;
    while (gk > 1 && (size_t)gk * M * N * sizeof(float) > workspace_bytes)
        gk /= 2;
    return gk;
}

size_t gemm_workspace_bytes(int M, int N, int K)
{
    const int gk = gemm_split(M, N, K, (size_t)-1);
    return gk > 1 ? (size_t)gk * M * N * sizeof(float) : 0;
}

hipError_t launch_gemm(const void *x, bool bf16, const uint8_t *wq, const uint16_t *scales,
                       float *y, int M, int N, int K, void *workspace, size_t workspace_bytes,
                       hipStream_t stream)
{
    const Plan plan = make_plan(K);
    const int gk = workspace ? gemm_split(M, N, K, workspace_bytes) : 1;
    const dim3 grid((N + GEMM_BN - 1) / GEMM_BN, (M + GEMM_BM - 1) / GEMM_BM, gk);
    float *out = gk > 1 ? (float *)workspace : y;
    if (bf16)
        hipLaunchKernelGGL(q4_gemm<true>, grid, dim3(256), 0, stream, (const uint16_t *)x, wq, scales,
                           out, M, N, K, plan, gk, gk > 1 ? 1 : 0);
    else
        hipLaunchKernelGGL(q4_gemm<false>, grid, dim3(256), 0, stream, (const uint16_t *)x, wq, scales,
                           out, M, N, K, plan, gk, gk > 1 ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || gk == 1)
        return e;
    const size_t mn = (size_t)M * N;
    hipLaunchKernelGGL(q4_tree_combine, dim3((unsigned)((mn + 255) / 256)), dim3(256), 0, stream,
                       (const float *)workspace, y, mn, gk);
    return hipGetLastError();
}

hipError_t launch_pack(const uint8_t *codes, uint8_t *wq, int N, int K, hipStream_t stream)
{
    const size_t chunks = (size_t)N * K / 32;
    hipLaunchKernelGGL(q4_pack_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, stream,
                       codes, wq, chunks);
    return hipGetLastError();
}

}  // namespace q4
