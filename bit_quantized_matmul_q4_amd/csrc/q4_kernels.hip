// q4_kernels.hip -- the Q4 linear kernels for gfx950 (MI355X).
//
// Two kernels compute y = x . dequant(Wq)^T, as the matrix-vector and
// matrix-matrix kernels of "Why Continuous Batching Slowed Down My LLM
// Inference Engine: A Metal Kernel Investigation" (section "Two Rows of
// Input, Two Different Kernels") do, but through one fixed reduction order
// (q4_device.hpp), so they return identical bits:
//
//  * q4_gemv: the weight-streaming kernel for small M.  A workgroup owns T
//    tiles of 16 output columns and a 16-row slice of the batch; its waves
//    split K into aligned runs of segments.  Each wave streams its run tile
//    by tile through a ring of D register stages (16-byte contiguous loads,
//    issued D quads ahead without branches), dequantizes in registers while
//    reading (the matrix-vector kernel's advantage the page names) and runs
//    the block dots on MFMA with all (<= 16) rows of x in the A operand.
//    The runs' subtree roots meet in LDS for the top of the pairwise tree.
//
//  * q4_gemm: the LDS-staged tile kernel for larger M.  A workgroup owns a
//    64 x 64 output tile; per quad it dequantizes the 64-column weight tile
//    into LDS once and stages the 64 x 128 activation tile, and four waves
//    run 2 x 2 MFMA tiles each from LDS.  K may be split across workgroups
//    (one subtree of segments each) when a workspace is given;
//    q4_tree_combine then joins the subtree roots in tree order.
//
//  * q4_pack_kernel: canonical codes and scales -> the tiled layout.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "q4_device.hpp"
#include "q4_launch.hpp"

namespace q4 {

// =================================================================== GEMV
// One ring stage: a quad of T column tiles as loaded.  Lane (g, c) holds per
// tile the B-operand dwords of the four block dots and the column's four
// scales, plus its A-operand slice (row slot c, k-slots 8g..8g+7) of each of
// the four blocks, shared by the T tiles.
template <int T>
struct GemvStage {
    u32x4 codes[T];
    u32x2 sc[T];
    u32x4 xa[4];
};

// Unconditional loads: the quad index is clamped by the caller, blocks past
// nb re-read block nb-1 of x (their MFMAs are skipped), and row slots past M
// re-read the last row (those outputs are never stored; an MFMA output
// element depends only on its own A row and B column).
template <int T>
__device__ __forceinline__ void gemv_load(GemvStage<T> &S, const uint8_t *wt, const uint16_t *st,
                                          size_t tile_bytes, size_t tile_scales,
                                          const uint16_t *xrow, int q, int nb)
{
#pragma unroll
    for (int t = 0; t < T; ++t) {
        S.codes[t] = *(const u32x4 *)(wt + t * tile_bytes + (size_t)q * 1024);
        S.sc[t] = *(const u32x2 *)(st + t * tile_scales + (size_t)q * 64);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        S.xa[i] = *(const u32x4 *)(xrow + (size_t)min(4 * q + i, nb - 1) * 32);
}

// R: accumulator registers that can hold real batch rows (min(rows, 4), a
// compile-time count so no per-register test reaches the hot loop).
// NQ: blocks in the quad (4, or fewer only for the last quad of K).
template <bool BF16, int T, int R>
__device__ __forceinline__ void gemv_compute(const GemvStage<T> &S, int nq, f32x4 (&p)[T])
{
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const uint32_t w[4] = {S.codes[t].x, S.codes[t].y, S.codes[t].z, S.codes[t].w};
        const uint32_t h[4] = {S.sc[t].x & 0xFFFFu, S.sc[t].x >> 16, S.sc[t].y & 0xFFFFu, S.sc[t].y >> 16};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i < nq) {
                const float d = half_bits_to_float(h[i]);
                const f32x4 s = blockdot<BF16>(S.xa[i], dequant8<BF16>(w[i]));
                p[t].x = __builtin_fmaf(d, s.x, p[t].x);
                if constexpr (R > 1)
                    p[t].y = __builtin_fmaf(d, s.y, p[t].y);
                if constexpr (R > 2)
                    p[t].z = __builtin_fmaf(d, s.z, p[t].z);
                if constexpr (R > 3)
                    p[t].w = __builtin_fmaf(d, s.w, p[t].w);
            }
        }
    }
}

// End of segment li of a run of L (1 or 4) segments: the pairwise tree
// of the run, written out.  After the run's last segment p holds the root.
// Each case is a real (uniform) branch: the empty asm keeps the compiler
// from turning the merges into per-quad selects.
template <int T, int L>
__device__ __forceinline__ void gemv_segment_done(int li, f32x4 (&p)[T], f32x4 (&s0)[T], f32x4 (&s1)[T])
{
    static_assert(L == 1 || L == 4, "runs of 1 or 4 segments");
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    if constexpr (L == 1)
        return;
    switch (li) {  // L == 4: ((p0 + p1) + (p2 + p3))
    case 0:
        asm volatile("");
#pragma unroll
        for (int t = 0; t < T; ++t) {
            s0[t] = p[t];
            p[t] = zero;
        }
        break;
    case 1:
        asm volatile("");
#pragma unroll
        for (int t = 0; t < T; ++t) {
            s1[t] = s0[t] + p[t];
            p[t] = zero;
        }
        break;
    case 2:
        asm volatile("");
#pragma unroll
        for (int t = 0; t < T; ++t) {
            s0[t] = p[t];
            p[t] = zero;
        }
        break;
    default:
        asm volatile("");
#pragma unroll
        for (int t = 0; t < T; ++t)
            p[t] = s1[t] + (s0[t] + p[t]);
        break;
    }
}

// grid = (ceil(N / (16 T)), ceil(M / 16)), block = 64 * Wc threads with
// Wc = S / L.  Wave w owns the aligned run of L segments starting at segment
// w L.  SHORT: K/32 is not a multiple of 4, so the last quad of K has fewer
// than four blocks.  Dynamic LDS: Wc * T * 16 * 17 floats (subtree roots).
template <bool BF16, int T, int D, int R, int L, bool SHORT>
__global__ __launch_bounds__(1024) void q4_gemv(const uint16_t *__restrict__ x,
                                                const uint8_t *__restrict__ wq,
                                                const uint16_t *__restrict__ scales,
                                                float *__restrict__ y, int M, int N, int K, Plan plan)
{
    extern __shared__ float red_lds[];  // [wave][tile][row slot][column slot (17)]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int Wc = blockDim.x >> 6;
    const int g = lane >> 4;   // lane group: k-slots 8g..8g+7, output rows 4g..4g+3
    const int c = lane & 15;   // column slot (B, D) and row slot (A)
    const int n16 = (N + 15) / 16;
    const int tile0 = blockIdx.x * T;
    const int m0 = blockIdx.y * 16;
    const int mrows = min(16, M - m0);
    const int G = plan.G;

    // tiles past the last one re-read the last tile (never stored)
    const size_t tile_bytes = (size_t)G * 1024;
    const size_t tile_scales = (size_t)G * 64;
    const int tfirst = min(tile0, n16 - 1);
    const uint8_t *wt = wq + (size_t)tfirst * tile_bytes + 16 * lane;
    const uint16_t *st = scales + (size_t)tfirst * tile_scales + 4 * c;
    size_t tstep_b = tile_bytes, tstep_s = tile_scales;
    if (tile0 + T > n16) {  // partial tile group at the end: all T tiles read the last one
        tstep_b = 0;
        tstep_s = 0;
    }
    const uint16_t *xrow = x + (size_t)(m0 + min(c, mrows - 1)) * K + 8 * g;

    const int seg0 = wave * L;
    const int q0 = (seg0 * G) >> plan.log2S;              // first quad of the run
    const int q1 = ((seg0 + L) * G) >> plan.log2S;        // end quad of the run
    const int qlast = q1 - 1;
    int li = 0;                                           // segment within the run
    int seg_end_q = ((seg0 + 1) * G) >> plan.log2S;       // end quad of the current segment

    f32x4 p[T], s0[T], s1[T];
#pragma unroll
    for (int t = 0; t < T; ++t)
        p[t] = (f32x4){0.f, 0.f, 0.f, 0.f};

    GemvStage<T> ring[D];
#pragma unroll
    for (int d = 0; d < D; ++d)
        gemv_load<T>(ring[d], wt, st, tstep_b, tstep_s, xrow, min(q0 + d, qlast), plan.nb);

    for (int q = q0; q < q1; q += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int qq = q + d;
            if (qq < q1) {
                if constexpr (SHORT)
                    gemv_compute<BF16, T, R>(ring[d], min(4, plan.nb - 4 * qq), p);
                else
                    gemv_compute<BF16, T, R>(ring[d], 4, p);
                if (qq + 1 == seg_end_q) {  // segment finished: fold into the run's subtree
                    gemv_segment_done<T, L>(li, p, s0, s1);
                    ++li;
                    seg_end_q = ((seg0 + li + 1) * G) >> plan.log2S;
                }
            }
            // refill this stage D quads ahead (clamped: past the run it
            // re-reads the run's last quad, an L2 hit)
            gemv_load<T>(ring[d], wt, st, tstep_b, tstep_s, xrow, min(qq + D, qlast), plan.nb);
        }
    }

#pragma unroll
    for (int t = 0; t < T; ++t) {
        float *r = red_lds + ((wave * T + t) * 16) * 17;
        r[(4 * g + 0) * 17 + c] = p[t].x;
        r[(4 * g + 1) * 17 + c] = p[t].y;
        r[(4 * g + 2) * 17 + c] = p[t].z;
        r[(4 * g + 3) * 17 + c] = p[t].w;
    }
    __syncthreads();

    // the Wc subtree roots -> the output; the whole workgroup shares the work
    for (int o = tid; o < T * 256; o += blockDim.x) {
        const int t = o >> 8;
        const int row = (o >> 4) & 15;
        const int col = o & 15;
        const int n = (tile0 + t) * 16 + col;
        if (row >= mrows || n >= N)
            continue;
        float v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
            v[j] = j < Wc ? red_lds[((j * T + t) * 16 + row) * 17 + col] : 0.f;
        y[(size_t)(m0 + row) * N + n] = tree_sum<16>(v, Wc) * 16.0f;
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
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int wr = wave >> 1, wc = wave & 1;
    const int g = lane >> 4, c = lane & 15;
    const int n0 = blockIdx.x * GEMM_BN;
    const int m0 = blockIdx.y * GEMM_BM;
    const int z = blockIdx.z;
    const int G = plan.G;
    const int n16 = (N + 15) / 16;

    const int L = plan.S / Gk;  // segments of this K-group (power of two)
    const int j0 = z * L;

    // weight staging: wave u stages column tile n0/16 + u (clamped; columns
    // past N carry unused data) -- lane (g, c) dequantizes its 16 bytes into
    // columns 16u + c, k-slots 32i + 8g.., i = 0..3
    const int wtile = min(n0 / 16 + wave, n16 - 1);
    const uint8_t *wsrc = wq + (size_t)wtile * G * 1024 + 16 * lane;
    const uint16_t *ssrc = scales + (size_t)wtile * G * 64 + 4 * c;
    // activation staging: thread -> (row st_r, block-in-quad st_q); rows past
    // M re-read row M-1 (never stored)
    const int st_r = tid >> 2;
    const int st_q = tid & 3;
    const uint16_t *xsrc_row = x + (size_t)min(m0 + st_r, M - 1) * K;

    f32x4 p[2][2];
    f32x4 stack[4][4];  // tree_push works on the four tiles as one array
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
            p[a][b] = (f32x4){0.f, 0.f, 0.f, 0.f};

    for (int li = 0; li < L; ++li) {
        const int seg = j0 + li;
        const int qb = (seg * G) >> plan.log2S;
        const int qe = ((seg + 1) * G) >> plan.log2S;
        for (int q = qb; q < qe; ++q) {
            const int nq = min(4, plan.nb - 4 * q);
            // ---- stage: dequantized weights, activations, scales
            {
                const u32x4 wv = *(const u32x4 *)(wsrc + (size_t)q * 1024);
                const u32x2 sv = *(const u32x2 *)(ssrc + (size_t)q * 64);
                const int bq = min(4 * q + st_q, plan.nb - 1);
                const u32x4 *xsrc = (const u32x4 *)(xsrc_row + (size_t)bq * 32);
                const u32x4 x0 = xsrc[0], x1 = xsrc[1], x2 = xsrc[2], x3 = xsrc[3];
                const int col = 16 * wave + c;
                *(u32x4 *)&ws[col][0 * 32 + 8 * g] = dequant8<BF16>(wv.x);
                *(u32x4 *)&ws[col][1 * 32 + 8 * g] = dequant8<BF16>(wv.y);
                *(u32x4 *)&ws[col][2 * 32 + 8 * g] = dequant8<BF16>(wv.z);
                *(u32x4 *)&ws[col][3 * 32 + 8 * g] = dequant8<BF16>(wv.w);
                if (g == 0) {
                    ds[0][col] = half_bits_to_float(sv.x & 0xFFFFu);
                    ds[1][col] = half_bits_to_float(sv.x >> 16);
                    ds[2][col] = half_bits_to_float(sv.y & 0xFFFFu);
                    ds[3][col] = half_bits_to_float(sv.y >> 16);
                }
                u32x4 *xdst = (u32x4 *)&xs[st_r][st_q * 32];
                xdst[0] = x0;
                xdst[1] = x1;
                xdst[2] = x2;
                xdst[3] = x3;
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
        // ---- segment done: fold into the K-group's subtree
        f32x4 cur[4] = {p[0][0], p[0][1], p[1][0], p[1][1]};
        if (!tree_push<4, 4>(stack, cur, li, L)) {
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    p[a][b] = (f32x4){0.f, 0.f, 0.f, 0.f};
        } else {
            p[0][0] = cur[0];
            p[0][1] = cur[1];
            p[1][0] = cur[2];
            p[1][1] = cur[3];
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
// One thread per (tile, quad, lane l = 16 g + c): gathers the 16 bytes of
// lane l (bytes 4g..4g+3 of blocks 4q..4q+3 of column 16t + c, packed from
// the canonical codes) and, for g == 0, the column's four scales.
__global__ __launch_bounds__(256) void q4_pack_kernel(const uint8_t *__restrict__ codes,
                                                      const uint16_t *__restrict__ scales_in,
                                                      uint8_t *__restrict__ wq,
                                                      uint16_t *__restrict__ scales_out, int N, int K,
                                                      size_t items)
{
    const size_t item = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (item >= items)
        return;
    const int nb = K / 32;
    const int G = (nb + 3) / 4;
    const int l = (int)(item & 63);
    const size_t tq = item >> 6;  // tile * G + quad
    const int q = (int)(tq % G);
    const int t = (int)(tq / G);
    const int g = l >> 4, c = l & 15;
    const int n = 16 * t + c;
    uint32_t out[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int b = 4 * q + i;
        uint32_t v = 0;
        if (n < N && b < nb) {
            const uint8_t *src = codes + (size_t)n * K + 32 * b + 8 * g;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t lo = src[2 * j] & 0x0Fu;
                const uint32_t hi = src[2 * j + 1] & 0x0Fu;
                v |= (lo | (hi << 4)) << (8 * j);
            }
        }
        out[i] = v;
    }
    *(u32x4 *)(wq + tq * 1024 + 16 * l) = (u32x4){out[0], out[1], out[2], out[3]};
    if (g == 0) {
        uint16_t sv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int b = 4 * q + i;
            sv[i] = (n < N && b < nb) ? scales_in[(size_t)n * nb + b] : (uint16_t)0;
        }
        uint16_t *dst = scales_out + tq * 64 + 4 * c;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dst[i] = sv[i];
    }
}

// ============================================================== launchers
// Launch shape of the GEMV: column tiles per workgroup (T), waves per
// workgroup (Wc: a power of two with S / Wc <= 4) and ring depth (D).  None
// of them changes the bits.  Q4_GEMV_T, Q4_GEMV_WAVES and Q4_GEMV_DEPTH
// override the heuristic (tuning only).
static int env_knob(const char *name)
{
    const char *v = getenv(name);
    return v ? atoi(v) : 0;
}

// L (segments per wave) is 4 or 1: Wc = S / 4 or S.
static void gemv_shape(int M, int N, const Plan &plan, int &T, int &L, int &D)
{
    (void)M;
    // measured on MI355X (7B shapes): wide N streams two tiles per wave in runs
    // of 4 segments; narrow N spreads one segment per wave over more waves
    const int tiles = (N + 15) / 16;
    const bool wide = plan.S >= 4 && tiles >= 1024;
    T = wide ? 2 : 1;
    D = 2;
    L = wide ? 4 : 1;
    static const int env_t = env_knob("Q4_GEMV_T");
    static const int env_l = env_knob("Q4_GEMV_RUN");
    static const int env_d = env_knob("Q4_GEMV_DEPTH");
    if (env_t == 1 || env_t == 2)
        T = env_t;
    if (env_d == 2 || env_d == 3)
        D = env_d;
    if (env_l == 1 || (env_l == 4 && plan.S >= 4))
        L = env_l;
}

// Every compile-time variant the launcher can pick: BF16 x T {1,2} x D
// {2,3} x R {1,2,4} x L {1,4} x SHORT.
struct GemvArgs {
    dim3 grid, block;
    size_t lds;
    hipStream_t stream;
    const uint16_t *x;
    const uint8_t *wq;
    const uint16_t *scales;
    float *y;
    int M, N, K;
    Plan plan;
};

template <bool BF16, int T, int D, int R, int L>
static void launch_gemv_v(const GemvArgs &a)
{
    if (a.plan.nb & 3)
        hipLaunchKernelGGL((q4_gemv<BF16, T, D, R, L, true>), a.grid, a.block, a.lds, a.stream, a.x, a.wq,
                           a.scales, a.y, a.M, a.N, a.K, a.plan);
    else
        hipLaunchKernelGGL((q4_gemv<BF16, T, D, R, L, false>), a.grid, a.block, a.lds, a.stream, a.x, a.wq,
                           a.scales, a.y, a.M, a.N, a.K, a.plan);
}

template <bool BF16, int T, int D, int R>
static void launch_gemv_l(int L, const GemvArgs &a)
{
    if (L == 4)
        launch_gemv_v<BF16, T, D, R, 4>(a);
    else
        launch_gemv_v<BF16, T, D, R, 1>(a);
}

template <bool BF16, int T, int D>
static void launch_gemv_r(int R, int L, const GemvArgs &a)
{
    if (R == 1)
        launch_gemv_l<BF16, T, D, 1>(L, a);
    else if (R == 2)
        launch_gemv_l<BF16, T, D, 2>(L, a);
    else
        launch_gemv_l<BF16, T, D, 4>(L, a);
}

template <bool BF16, int T>
static void launch_gemv_d(int D, int R, int L, const GemvArgs &a)
{
    // two tiles per wave with a 3-deep ring would spill registers: not built
    if (T == 1 && D == 3)
        launch_gemv_r<BF16, T, T == 1 ? 3 : 2>(R, L, a);
    else
        launch_gemv_r<BF16, T, 2>(R, L, a);
}

hipError_t launch_gemv(const void *x, bool bf16, const uint8_t *wq, const uint16_t *scales,
                       float *y, int M, int N, int K, hipStream_t stream)
{
    const Plan plan = make_plan(K);
    int T, L, D;
    gemv_shape(M, N, plan, T, L, D);
    const int Wc = plan.S / L;
    GemvArgs a;
    a.grid = dim3((N + 16 * T - 1) / (16 * T), (M + 15) / 16);
    a.block = dim3(64 * Wc);
    a.lds = (size_t)Wc * T * 16 * 17 * sizeof(float);
    a.stream = stream;
    a.x = (const uint16_t *)x;
    a.wq = wq;
    a.scales = scales;
    a.y = y;
    a.M = M;
    a.N = N;
    a.K = K;
    a.plan = plan;
    // every 16-row slice but a last short one has 16 rows; 3 rows use R = 4
    const int R = M >= 3 ? 4 : M;
    if (bf16) {
        if (T == 2)
            launch_gemv_d<true, 2>(D, R, L, a);
        else
            launch_gemv_d<true, 1>(D, R, L, a);
    } else {
        if (T == 2)
            launch_gemv_d<false, 2>(D, R, L, a);
        else
            launch_gemv_d<false, 1>(D, R, L, a);
    }
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

size_t packed_code_bytes(int N, int K) { return (size_t)((N + 15) / 16) * ((K / 32 + 3) / 4) * 1024; }

size_t packed_scale_bytes(int N, int K) { return (size_t)((N + 15) / 16) * ((K / 32 + 3) / 4) * 128; }

hipError_t launch_pack(const uint8_t *codes, const uint16_t *scales_in, uint8_t *wq, uint16_t *scales_out,
                       int N, int K, hipStream_t stream)
{
    const size_t items = packed_code_bytes(N, K) / 16;
    hipLaunchKernelGGL(q4_pack_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, codes,
                       scales_in, wq, scales_out, N, K, items);
    return hipGetLastError();
}

}  // namespace q4
