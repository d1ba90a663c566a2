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
//    the block dots on MFMA with all (<= 16) rows of x in the A operand
//    (x staged in LDS, loaded in the slot layout that gives one MFMA the
//    corrections of a whole quad, or loaded with the ring: see XM_RING).
//    The runs' subtree roots meet in LDS for the top of the pairwise tree.
//
//  * q4_gemv_seg: the same kernel's form for wide N (more than 256 or 512
//    column tiles, see seg_shape): a workgroup of 16 waves owns a run of
//    column tiles, wave j owns segment j of all of them and holds that
//    segment of x in registers, so the workgroup reads x once.
//
//  * q4_gemm_ws: the matrix-matrix kernel for larger M.  A workgroup of
//    4..8 waves owns an output unit of 16 or 32 rows by one column tile per
//    wave; each wave streams its tile's codes and scales through a register
//    ring and reads the unit's activations from a two-stage LDS ring the
//    waves fill through registers.  K may be split across workgroups (one
//    subtree of segments each) when a workspace is given; q4_tree_combine
//    then joins the subtree roots in tree order.
//
//  * q4_pack_kernel: canonical codes and scales -> the tiled layout.
//
//  * q4_quantize_kernel: dense weights -> canonical codes and scales.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "q4_device.hpp"
#include "q4_launch.hpp"

namespace q4 {

// =================================================================== GEMV
// Buffer resource over a wave-uniform base, with the exact byte range of the
// data a wave may read.  Every load below passes its whole offset (the
// lane's part plus the running stream position) as the vector offset, which
// the raw-buffer range check covers: a load whose vector offset is at or
// past the range returns zeros and makes no memory access.  The kernels use
// that on purpose for refills past a stream's end and for row slots past the
// batch, and pass a scalar offset of zero everywhere, so no read can leave
// its buffer whether or not the check also counts the scalar offset.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes = 0xFFFFFFFFu)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Cache policy of the code and scale loads: the non-temporal hint (nt), for
// data a call reads once (or, in the matrix-matrix kernel, once per row
// unit).  Measured on MI355X against the default policy in back-to-back
// calls: the matrix-vector kernels get 5-9% faster per launch on every
// 7B-shaped projection at one to eight rows (k_proj 4.87 -> 4.52 us, gate
// 11.5 -> 10.9 us, down 10.9 -> 9.9 us at one row), the matrix-matrix
// kernel 0.5 us faster on q_proj and k_proj and unchanged on the larger
// matrices.  x keeps the default: every workgroup rereads it from L2.
constexpr int kWeightLoadPolicy = 2;

// One ring stage: one tile-quad of the wave's stream as loaded.  Lane (g, c)
// holds the B-operand dwords of the quad's four block dots, its column's four
// scales and its A-operand slice (row slot c, k-slots 8g..8g+7) of the four
// blocks of x.
constexpr int GEMV_TPS_MAX = 8;  // column tiles per stream (outputs staged in LDS)

struct GemvStage {
    u32x4 w;
    u32x2 s;
    u32x4 xa[4];
};

// R: accumulator components that can hold real batch rows (min(rows, 4),
// compile-time).  nq: blocks in the quad (4 except a short last quad).
template <bool BF16, int R, bool SHORT>
__device__ __forceinline__ void gemv_quad(const GemvStage &st, const u32x4 (&xa)[4], int nq, const Dequant<BF16> &dq,
                                          float (&p)[R])
{
    const uint32_t w[4] = {st.w.x, st.w.y, st.w.z, st.w.w};
    const uint32_t h[4] = {st.s.x & 0xFFFFu, st.s.x >> 16, st.s.y & 0xFFFFu, st.s.y >> 16};
    // the block dots first, so their matrix-core latencies overlap
    f32x4 C[4], D[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        C[i] = correction<BF16>(xa[i], dq);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        D[i] = block_dot<BF16>(xa[i], dq(w[i]), C[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (!SHORT || i < nq) {
            const float d = half_bits_to_float(h[i]);
#pragma unroll
            for (int r = 0; r < R; ++r)
                p[r] = __builtin_fmaf(d, D[i][r], p[r]);
        }
    }
}

// The block values of a quad (bv[i][r]: block i, accumulator row r), the
// part of gemv_quad before its scale-accumulates.
template <bool BF16, int R>
__device__ __forceinline__ void gemv_block_values(const GemvStage &st, const u32x4 (&xa)[4], const Dequant<BF16> &dq,
                                                  float (&bv)[4][R])
{
    const uint32_t w[4] = {st.w.x, st.w.y, st.w.z, st.w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x4 D = block_dot<BF16>(xa[i], dq(w[i]), correction<BF16>(xa[i], dq));
#pragma unroll
        for (int r = 0; r < R; ++r)
            bv[i][r] = D[r];
    }
}

// gemv_quad with the quad's corrections already computed (Cq[i]: block
// i's), for waves that hold their x for many tiles: the correction depends
// on x only, so the same instruction on the same operands gives the same
// bits wherever it runs.
template <bool BF16, int R, bool SHORT>
__device__ __forceinline__ void gemv_quad_pre(const GemvStage &st, const u32x4 (&xa)[4], const f32x4 (&Cq)[4], int nq,
                                              const Dequant<BF16> &dq, float (&p)[R])
{
    const uint32_t w[4] = {st.w.x, st.w.y, st.w.z, st.w.w};
    const uint32_t h[4] = {st.s.x & 0xFFFFu, st.s.x >> 16, st.s.y & 0xFFFFu, st.s.y >> 16};
    f32x4 D[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        D[i] = block_dot<BF16>(xa[i], dq(w[i]), Cq[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (!SHORT || i < nq) {
            const float d = half_bits_to_float(h[i]);
#pragma unroll
            for (int r = 0; r < R; ++r)
                p[r] = __builtin_fmaf(d, D[i][r], p[r]);
        }
    }
}

// One batch row per lane group (R = 1) with x in the slot layout: A row slot
// 4 i + j holds batch row i's block j of the quad (lane (g, 4 i + j) holds
// that block's k-slots 8 g .. 8 g + 7; the loads of XM_SLOT, or one read of
// x staged in LDS).  One correction MFMA then gives every (row, block) pair
// its correction in its own slot, and block j's dot runs on the same A
// operand with that accumulator input: row i's value lands in slot 4 i + j,
// component j of lane group i.  An MFMA result element depends only on its
// own A row, B column and accumulator input, so these are the bits of the
// one-block-per-dot form (same instruction, same operands), with 5 MFMAs a
// quad instead of 8 and no gathering of x.
template <bool BF16, bool SHORT>
__device__ __forceinline__ void gemv_quad_slots(const u32x4 &w, const u32x2 &s, const u32x4 &a, int nq,
                                                const Dequant<BF16> &dq, float (&p)[1])
{
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    const uint32_t h[4] = {s.x & 0xFFFFu, s.x >> 16, s.y & 0xFFFFu, s.y >> 16};
    const f32x4 C = correction<BF16>(a, dq);
    f32x4 D[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        D[i] = block_dot<BF16>(a, dq(wd[i]), C);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (!SHORT || i < nq)
            p[0] = __builtin_fmaf(half_bits_to_float(h[i]), D[i][i], p[0]);
}

// The block values of a quad in the slot layout (bv[i][0]: block i).
template <bool BF16>
__device__ __forceinline__ void gemv_block_values_slots(const u32x4 &w, const u32x4 &a, const Dequant<BF16> &dq,
                                                        float (&bv)[4][1])
{
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    const f32x4 C = correction<BF16>(a, dq);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        bv[i][0] = block_dot<BF16>(a, dq(wd[i]), C)[i];
}

// Two batch rows per lane group (R = 2) in the slot layout of XM_SLOT's
// loads: operand a holds blocks 0 and 1 of the quad, operand b blocks 2 and
// 3, A row slot 4 i + k holding row i + 4 (k & 1) of block k >> 1 (of the
// pair).  One correction MFMA per operand covers its four (row, block)
// pairs; the first block of a pair lands in components 0 (row i) and 1 (row
// i + 4) of lane group i, the second in components 2 and 3.  6 MFMAs a quad
// instead of 8, the same bits (as in gemv_quad_slots).
template <bool BF16, bool SHORT>
__device__ __forceinline__ void gemv_quad_slots2(const u32x4 &w, const u32x2 &s, const u32x4 &a, const u32x4 &b,
                                                 int nq, const Dequant<BF16> &dq, float (&p)[2])
{
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    const uint32_t h[4] = {s.x & 0xFFFFu, s.x >> 16, s.y & 0xFFFFu, s.y >> 16};
    const f32x4 Ca = correction<BF16>(a, dq), Cb = correction<BF16>(b, dq);
    f32x4 D[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        D[i] = block_dot<BF16>(i < 2 ? a : b, dq(wd[i]), i < 2 ? Ca : Cb);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (!SHORT || i < nq) {
            const float d = half_bits_to_float(h[i]);
            p[0] = __builtin_fmaf(d, D[i][2 * (i & 1)], p[0]);
            p[1] = __builtin_fmaf(d, D[i][2 * (i & 1) + 1], p[1]);
        }
    }
}

// The block values of a quad in the two-row slot layout (bv[i][r]).
template <bool BF16>
__device__ __forceinline__ void gemv_block_values_slots2(const u32x4 &w, const u32x4 &a, const u32x4 &b,
                                                         const Dequant<BF16> &dq, float (&bv)[4][2])
{
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    const f32x4 Ca = correction<BF16>(a, dq), Cb = correction<BF16>(b, dq);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x4 v = block_dot<BF16>(i < 2 ? a : b, dq(wd[i]), i < 2 ? Ca : Cb);
        bv[i][0] = v[2 * (i & 1)];
        bv[i][1] = v[2 * (i & 1) + 1];
    }
}

// The wave's stream is a contiguous run of tile-quads: quad i of the stream
// sits at code byte 1024 i and scale byte 128 i from the wave's base, and is
// quad q0 + (i mod RQ) of K.  The code and scale resources span exactly the
// stream, so the ring's refills past the end (vector offsets at or past the
// range) return zero without a memory access, with no clamp or test.  x
// blocks past nb (a short last quad) read whatever follows (the next row, or
// zero past the slice); their block dots are skipped.
struct GemvStream {
    __amdgpu_buffer_rsrc_t w, s, x;
    uint32_t w_lane, s_lane, x_lane;  // per-lane byte offsets
    uint32_t xw_lane[2];              // XM_SLOT: the (row, block) pairs of the lane's slots
    uint32_t w_off, s_off;            // scalar offsets of the next refill
};

// Where the matrix-vector kernel's A operands (x) come from.
//  XM_RING: loaded with each ring stage in the A-operand layout: four
//    16-byte loads a lane (one per block), whatever the row count.
//  XM_LDS: the workgroup's rows copied into LDS once, before the loop (the
//    split form reads them in the slot layout).
//  XM_SLOT: up to 8 rows, loaded with each ring stage in the slot layout
//    (gemv_quad_slots, gemv_quad_slots2): the lanes of the row slots that
//    hold no batch row load other blocks of the rows, so that each load
//    reads whole 128-byte lines and the A operands need no gathering.
//    Measured on MI355X against rows loaded in row order and turned into the
//    A-operand layout through a per-wave LDS slot: q_proj at 1 / 8 rows 4.34
//    / 4.90 -> 4.11 / 4.74 us, down_proj at 2 rows 10.22 -> 9.34 us; and
//    that slot form against XM_RING at 8 rows, down_proj 16.0 -> 13.3 us.
enum : int { XM_RING = 0, XM_LDS = 1, XM_SLOT = 3 };

// Keeps the ring's loads in program order relative to their uses: the empty
// statement (no instructions) with a memory clobber stops IR-level motion,
// the scheduling barrier stops the machine scheduler.
__device__ __forceinline__ void issue_fence()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Loads one stage: the next quad of the stream and, unless x is staged in
// LDS (XM_LDS), the x of quad x_off / 256 (x_off >= the slice size for a
// refill past the stream's end): the four A-operand blocks (XM_RING) or NW
// slot-layout operands (XM_SLOT, into xa[0 .. NW - 1]).
template <int XM, int NW>
__device__ __forceinline__ void gemv_load_x(GemvStage &st, GemvStream &in, uint32_t x_off)
{
    if constexpr (XM == XM_RING) {
#pragma unroll
        for (int b = 0; b < 4; ++b)
            st.xa[b] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(in.x, in.x_lane + 64u * b + x_off, 0, 0));
    } else if constexpr (XM == XM_SLOT) {
#pragma unroll
        for (int j = 0; j < NW; ++j)
            st.xa[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(in.x, in.xw_lane[j] + x_off, 0, 0));
    }
}

template <int XM, int NW, bool LS = true, bool LX = true>
__device__ __forceinline__ void gemv_load(GemvStage &st, GemvStream &in, uint32_t x_off)
{
    st.w = __builtin_bit_cast(u32x4,
                              __builtin_amdgcn_raw_buffer_load_b128(in.w, in.w_lane + in.w_off, 0, kWeightLoadPolicy));
    if constexpr (LS)  // else the scales come in groups (q4_gemv)
        st.s = __builtin_bit_cast(u32x2,
                                  __builtin_amdgcn_raw_buffer_load_b64(in.s, in.s_lane + in.s_off, 0, kWeightLoadPolicy));
    if constexpr (!LX) {
    } else if constexpr (XM == XM_RING) {
#pragma unroll
        for (int b = 0; b < 4; ++b)
            st.xa[b] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(in.x, in.x_lane + 64u * b + x_off, 0, 0));
    } else if constexpr (XM == XM_SLOT) {
        static_assert(NW == 1 || NW == 2, "XM_SLOT holds up to 8 rows");
#pragma unroll
        for (int j = 0; j < NW; ++j)
            st.xa[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(in.x, in.xw_lane[j] + x_off, 0, 0));
    }
    in.w_off += 1024;
    in.s_off += 128;
}

// A-operand slice of quad q from the x rows staged in LDS (lane row base
// xrow, 16 g already added): four 16-byte reads.
__device__ __forceinline__ void gemv_x_lds(u32x4 (&xa)[4], const uint8_t *xrow, int q)
{
#pragma unroll
    for (int b = 0; b < 4; ++b)
        xa[b] = *(const u32x4 *)(xrow + 256 * q + 64 * b);
}

// Row slots of a 16-row slice.  Batch row m sits in A-operand row slot
// 4 (m mod 4) + m / 4, so that element i of a lane group g's accumulator
// (D row slot 4 g + i) holds batch row 4 i + g: the rows spread over the four
// lane groups and a lane holds only ceil(rows / 4) of them (R = 1 up to 4
// rows, 2 up to 8).  A row's block dot does not depend on its slot, so the
// bits do not change with the placement.
__device__ __forceinline__ int slot_row(int s) { return 4 * (s & 3) + (s >> 2); }

// Bytes of LDS a row of x takes when staged: padded by 16 so that rows start
// in different banks.
__host__ __device__ constexpr uint32_t gemv_xrow_bytes(int K) { return (uint32_t)K * 2u + 16u; }

// The matrices one launch of a matrix-vector kernel runs (one, or a group
// that shares x, M and K): passed by value in the kernel arguments.
// NM: the table's size, 1 for a single matrix (a larger argument block
// measurably slows every launch) or kGroupMax.
constexpr int kGroupMax = 8;
template <int NM>
struct MatrixItems {
    int count;
    int wg_end[NM];  // workgroups (grid x) of matrices 0..i, cumulative
    const uint8_t *wq[NM];
    const uint16_t *scales[NM];
    float *y[NM];
    int N[NM];
};

// The workgroup's matrix (workgroups wg_end[i - 1] .. wg_end[i] - 1 run
// matrix i) and the first workgroup of that matrix, chosen by selects on
// uniform values: an indexed read of the argument block could be copied to
// scratch memory.
struct MatrixSel {
    const uint8_t *wq;
    const uint16_t *scales;
    float *y;
    int N, wg0;
};
template <int NM>
__device__ __forceinline__ MatrixSel select_matrix(const MatrixItems<NM> items)
{
    int it = 0;
#pragma unroll
    for (int i = 1; i < NM; ++i)
        if (i < items.count && (int)blockIdx.x >= items.wg_end[i - 1])
            it = i;
    MatrixSel m{items.wq[0], items.scales[0], items.y[0], items.N[0], 0};
#pragma unroll
    for (int i = 1; i < NM; ++i)
        if (i == it) {
            m.wq = items.wq[i];
            m.scales = items.scales[i];
            m.y = items.y[i];
            m.N = items.N[i];
            m.wg0 = items.wg_end[i - 1];
        }
    return m;
}

// grid = (streams / 4, or column tiles summed over the matrices of `items`,
// ceil(M / 16)); SPLIT: a workgroup's matrix is the one whose range of
// workgroup ids holds it, and its tiles count from that range's start; the
// streaming form runs items' first matrix only.
//  SPLIT = false: block = 256; each wave streams `tps` consecutive column
//    tiles over all of K (one run of S segments) and stores each tile's
//    outputs itself.
//  SPLIT = true: block = 64 TW W <= 512 with W = S / L; the workgroup owns TW
//    column tiles, wave (slot, run) streams run `run` (segments run L ..
//    run L + L - 1) of tile slot `slot`; each tile's W run roots meet in LDS
//    for the top of the pairwise tree.
//  XM (see XM_RING, XM_LDS, XM_SLOT): where the A operands come from.
//  XF: 0, x loaded with each stage's codes; 1 (one row), x first in the
//    prefill; 2 (bf16 split form, up to 8 rows, every run held whole by the
//    prefill), x first and the corrections of all stages computed while the
//    codes are still in flight.
// Dynamic LDS: [4 waves][tps tiles][16][16] tile roots (SPLIT = false), then
// (XM_LDS) min(M, 16) rows of gemv_xrow_bytes(K) bytes and 256 bytes of
// slack.
template <bool BF16, int R, int D, bool SHORT, bool SPLIT, int XM, int NM, int XF>
__global__ __launch_bounds__(SPLIT ? 512 : 256) void q4_gemv(const uint16_t *__restrict__ x, MatrixItems<NM> items,
                                                              int M, int K, Plan plan, int L, int tps)
{
    // (the streaming form runs one matrix)
    const MatrixSel sel =
        SPLIT ? select_matrix(items) : MatrixSel{items.wq[0], items.scales[0], items.y[0], items.N[0], 0};
    const uint8_t *__restrict__ wq = sel.wq;
    const uint16_t *__restrict__ scales = sel.scales;
    float *__restrict__ y = sel.y;
    const int N = sel.N;
    const int wgx = (int)blockIdx.x - sel.wg0;  // the workgroup within its matrix
    constexpr bool XL = XM == XM_LDS;
    // SPLIT: the run roots, [wave][row slot][column slot (17)].  Otherwise the
    // stream's tile roots (dynamic LDS): a store inside the streaming loop
    // would make every wait on the ring drain the whole ring (loads and
    // stores share one counter), so y is written after it.
    __shared__ float red[SPLIT ? 8 * 16 * 17 : 1];
    extern __shared__ __attribute__((aligned(16))) float dyn_lds[];
    float *ystage = dyn_lds;
    uint8_t *xlds = (uint8_t *)(dyn_lds + (SPLIT ? 0 : 4 * tps * 256));
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;  // k-slots 8g..8g+7 (A, B); batch rows g, g+4, .. (D)
    const int c = lane & 15;  // row slot (A); column slot (B, D)
    const int n16 = (N + 15) / 16;
    const int G = plan.G;
    const int m0 = blockIdx.y * 16;
    const int mrows = min(16, M - m0);

    // SPLIT: the workgroup's waves are TW tile slots by W runs (wave = slot W
    // + run); W = S / L is a power of two
    const int log2W = SPLIT ? plan.log2S - (31 - __builtin_clz(L)) : 0;
    int t0, ntiles, run;
    if constexpr (SPLIT) {
        const int TW = (blockDim.x >> 6) >> log2W;
        t0 = wgx * TW + (wave >> log2W);
        ntiles = t0 < n16 ? 1 : 0;  // 0: a spare slot of the last workgroup
        run = wave & ((1 << log2W) - 1);
    } else {
        t0 = (wgx * 4 + wave) * tps;
        ntiles = max(0, min(tps, n16 - t0));  // 0: a spare wave of the last workgroup
        run = 0;
        if (!XL && ntiles == 0)
            return;  // no barrier follows in this form
    }
    const int seg0 = run * L;
    const int q0 = (seg0 * G) >> plan.log2S;
    const int q1 = ((seg0 + L) * G) >> plan.log2S;
    const int total = ntiles * (q1 - q0);

    const uint32_t x_bytes = (uint32_t)mrows * (uint32_t)K * 2u;
    GemvStream in;
    in.w = buffer_rsrc(wq + ((size_t)min(t0, n16 - 1) * G + q0) * 1024, (uint32_t)total * 1024u);
    in.s = buffer_rsrc(scales + ((size_t)min(t0, n16 - 1) * G + q0) * 64, (uint32_t)total * 128u);
    if constexpr (XF != 0) {
        // x's loads stay where they are written (the compiler may otherwise
        // move loads of a read-only argument down to their first use, here
        // behind the wait for the prefill)
        const uint16_t *xs_base = x + (size_t)m0 * K;
        asm volatile("" : "+s"(xs_base));
        in.x = buffer_rsrc(xs_base, x_bytes);
    } else {
        in.x = buffer_rsrc(x + (size_t)m0 * K, x_bytes);
    }
    in.w_lane = 16u * lane;
    in.s_lane = 8u * c;
    // row slots past the batch read nothing (an offset past the resource's
    // range returns zeros without a memory access); they only feed output
    // rows that are never stored
    const int xr = slot_row(c);  // the batch row of A row slot c
    in.x_lane = xr < mrows ? (uint32_t)xr * (uint32_t)K * 2u + 16u * g : x_bytes;
    if constexpr (XM == XM_SLOT) {
        // the slot layout: lane (g, 4 i + k) loads, for operand j, batch row
        // i (R = 1) or i + 4 (k & 1) (R = 2) and block k (R = 1) or 2 j +
        // (k >> 1) (R = 2), k-slots 8 g .. 8 g + 7
        const int pc = R == 1 ? (c & ~3) : (c & ~2);
        const int qr = slot_row(pc);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int b = R == 1 ? (c & 3) : 2 * j + ((c >> 1) & 1);
            in.xw_lane[j] = qr < mrows ? (uint32_t)qr * (uint32_t)K * 2u + 64u * (uint32_t)b + 16u * g : x_bytes;
        }
    }
    in.w_off = 0;
    in.s_off = 0;

    // XL: x is copied into LDS, 16 bytes per thread and step, in rounds of 8
    // loads so that each round costs one memory round trip.  The first
    // round's loads go out ahead of the ring's prefill: x is what every wave
    // needs first, and behind the prefill they would wait for the first
    // stages of the whole grid.  Chunks past the rows fall outside x's range
    // (zero, no memory access) and land in the slack past the rows: with a
    // conditional store the compiler sinks the load into it, behind a wait
    // for the whole prefill.
    const int cpr = K / 8;  // 16-byte chunks per row
    const int nch = mrows * cpr;
    u32x4 xv[8];
    auto x_round_load = [&](int i0) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint32_t i = (uint32_t)(i0 + u * (int)blockDim.x + (int)threadIdx.x);
            xv[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(in.x, i * 16u, 0, 0));
        }
    };
    auto x_round_store = [&](int i0) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = min(i0 + u * (int)blockDim.x + (int)threadIdx.x, nch);
            const int r = i / cpr;  // mrows for the slack
            *(u32x4 *)(xlds + (uint32_t)r * gemv_xrow_bytes(K) + (uint32_t)(i - r * cpr) * 16u) = xv[u];
        }
    };
    if constexpr (XL) {
        x_round_load(0);
        issue_fence();
    }

    GemvStage ring[D];
    int ql = q0;     // quad of the next stage to load
    int left = total;  // loads left that the stream uses
    // Scale groups (four-stage rings): one 8-byte load a lane for four
    // consecutive stream quads, the lanes of row g loading quad g's column
    // scales; each stage takes its quad's from that row by ds_bpermute (as in
    // the segment form).  Groups past the stream read nothing.
    constexpr bool SG = D == 4;
    uint32_t sg_off = 0;
    auto load_group = [&]() -> u32x2 {
        const u32x2 v = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_raw_buffer_load_b64(in.s, in.s_lane + 128u * g + sg_off, 0, kWeightLoadPolicy));
        sg_off += 512;
        return v;
    };
    u32x2 sg_cur{0u, 0u}, sg_next{0u, 0u};
    if constexpr (SG) {
        sg_next = load_group();
        issue_fence();
    }
    // XF != 0: the prefill's x first, then its codes.  Otherwise the x of
    // each prefill stage is written with its codes but the compiler issues it
    // after the wait below (see XF), one round trip to cache later.  Measured
    // on MI355X: at one row x first is faster (down_proj 10.8 -> 9.8 us);
    // from two rows, without XF = 2's corrections ahead, x after the codes
    // (k_proj at 8 rows 5.2 -> 4.7 us).
    if constexpr (XF != 0) {
        int qx = ql, lx = left;
#pragma unroll
        for (int d = 0; d < D; ++d) {
            gemv_load_x<XM, R>(ring[d], in, lx > 0 ? 256u * qx : x_bytes);
            qx = qx + 1 == q1 ? q0 : qx + 1;
            --lx;
        }
        issue_fence();
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {  // in stage order (see the refill below)
        gemv_load<XM, R, !SG, XF == 0>(ring[d], in, left > 0 ? 256u * ql : x_bytes);
        ql = ql + 1 == q1 ? q0 : ql + 1;
        --left;
        issue_fence();
    }
    const uint8_t *xrow = xlds + (uint32_t)min(xr, mrows - 1) * gemv_xrow_bytes(K) + 16 * g;
    // x in the slot layout (gemv_quad_slots, gemv_quad_slots2): the loads of
    // XM_SLOT as they are, or (one row per lane group) one read of the staged
    // rows (rows past the batch read the last row: their slots are never
    // stored)
    constexpr bool SLOTS = R == 1 && (XM == XM_SLOT || XM == XM_LDS);
    constexpr bool SLOTS2 = R == 2 && XM == XM_SLOT;
    const uint8_t *xslot =
        xlds + (uint32_t)min(c >> 2, mrows - 1) * gemv_xrow_bytes(K) + 64u * (uint32_t)(c & 3) + 16u * (uint32_t)g;
    if constexpr (XL) {
        x_round_store(0);
        for (int i0 = 8 * (int)blockDim.x; i0 < nch; i0 += 8 * (int)blockDim.x) {
            x_round_load(i0);
            x_round_store(i0);
        }
        __syncthreads();
    }
    // A split-form run that the prefill holds whole (total <= D: q, k and v
    // of the 7B set) is computed from the ring without a loop (below).
    const bool whole = SPLIT && !XL && (R == 1 || XF == 2) && total <= D;
    // The compiler may reorder the prefill's loads (it clusters loads from
    // one base).  Waiting for all of them here costs little (they were issued
    // together and the first compute needs the first of them) and keeps that
    // order from pessimising every wait of the loop, whose header merges the
    // prefill's pending loads with the refills'.  (XF = 2: the compiler's
    // own waits, x before the codes.)
    if (!(XF == 2 && whole))
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    const Dequant<BF16> dq;
    // accumulators: the R rows a lane can hold (batch rows g + 4 r, r < R)
    float p[R], root[R];
    TreeStack<R, float> stack;
#pragma unroll
    for (int r = 0; r < R; ++r)
        p[r] = root[r] = 0.f;
    int qc = q0;  // quad being computed
    int t = 0;    // its tile, counted from t0
    int li = 0;   // segment within the run
    int seg_end = ((seg0 + 1) * G) >> plan.log2S;
    u32x4 xb[2][4];  // XL: x of the quad being computed and of the next
    if constexpr (XL) {
        if constexpr (SLOTS)
            xb[0][0] = *(const u32x4 *)(xslot + 256u * (uint32_t)q0);
        else
            gemv_x_lds(xb[0], xrow, q0);
    }
    // after quad qc's scale-accumulates: at a segment's end, fold it into the
    // run's subtree
    auto finish_quad = [&](int qn) {
        if (qc + 1 == seg_end) {
            if (stack.push(p, li, L)) {
                if constexpr (SPLIT) {
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        root[r] = p[r];
                } else {  // the tile's root, kept in LDS until the stream ends
                    float *o = ystage + ((wave * tps + t) * 16 + g) * 16 + c;
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        o[64 * r] = p[r];
                    ++t;
                }
                li = 0;
            } else {
                ++li;
            }
            seg_end = ((seg0 + li + 1) * G) >> plan.log2S;
#pragma unroll
            for (int r = 0; r < R; ++r)
                p[r] = 0.f;
        }
        qc = qn;
    };
    // A run held whole: every stage's A operands and block dots first, so
    // that the stages' LDS and matrix-core latencies overlap (such runs often
    // have a SIMD to themselves), then the scale-accumulates in order.
    // Measured on MI355X: a stage costs ~0.25 us of latency one after the
    // other; up to 4 rows this takes q_proj 4.9 -> 4.6 us, k_proj 4.3 -> 4.0
    // us and 896 x 896 3.3 -> 3.2 us (at 8 rows the registers it needs cost
    // more than it saves, without XF = 2).  XF = 2 loads x first and computes
    // the corrections before the codes arrive, up to 8 rows (q_proj at 1 / 4
    // / 8 rows 4.55 / 4.64 / 5.32 -> 4.34 / 4.41 / 4.85 us, k_proj 3.92 /
    // 4.17 / 4.65 -> 3.79 / 3.99 / 4.46 us); it has its own instantiation, as
    // the registers it holds (the A operands and corrections of all stages)
    // slow the longer runs of down_proj by 4%.
    if (whole) {
        if constexpr (SG) {
            sg_cur = sg_next;
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int src = (16 * d + c) << 2;
                ring[d].s.x = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)sg_cur.x);
                ring[d].s.y = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)sg_cur.y);
            }
        }
        float bv[D][4][R];
        // XF = 2: all stages' corrections, then their block dots once the
        // codes are there (guarded: only the stages the run holds)
        auto ahead = [&](auto guarded) {
            constexpr bool GD = decltype(guarded)::value;
            if constexpr (SLOTS) {  // one correction a stage
                f32x4 C1[D];
#pragma unroll
                for (int d = 0; d < D; ++d)
                    if (!GD || d < total)
                        C1[d] = correction<BF16>(ring[d].xa[0], dq);
                issue_fence();
#pragma unroll
                for (int d = 0; d < D; ++d) {
                    if (!GD || d < total) {
                        const uint32_t w[4] = {ring[d].w.x, ring[d].w.y, ring[d].w.z, ring[d].w.w};
#pragma unroll
                        for (int b = 0; b < 4; ++b)
                            bv[d][b][0] = block_dot<BF16>(ring[d].xa[0], dq(w[b]), C1[d])[b];
                    }
                }
                return;
            }
            if constexpr (SLOTS2) {  // two corrections a stage
                f32x4 C2[D][2];
#pragma unroll
                for (int d = 0; d < D; ++d)
                    if (!GD || d < total) {
                        C2[d][0] = correction<BF16>(ring[d].xa[0], dq);
                        C2[d][1] = correction<BF16>(ring[d].xa[1], dq);
                    }
                issue_fence();
#pragma unroll
                for (int d = 0; d < D; ++d) {
                    if (!GD || d < total) {
                        const uint32_t w[4] = {ring[d].w.x, ring[d].w.y, ring[d].w.z, ring[d].w.w};
#pragma unroll
                        for (int b = 0; b < 4; ++b) {
                            const f32x4 v = block_dot<BF16>(ring[d].xa[b >> 1], dq(w[b]), C2[d][b >> 1]);
                            bv[d][b][0] = v[2 * (b & 1)];
                            bv[d][b][1] = v[2 * (b & 1) + 1];
                        }
                    }
                }
                return;
            }
            u32x4 xa[D][4];
            f32x4 C[D][4];
#pragma unroll
            for (int d = 0; d < D; ++d) {
                if (!GD || d < total) {
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        xa[d][b] = ring[d].xa[b];
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        C[d][b] = correction<BF16>(xa[d][b], dq);
                }
            }
            issue_fence();
#pragma unroll
            for (int d = 0; d < D; ++d) {
                if (!GD || d < total) {
                    const uint32_t w[4] = {ring[d].w.x, ring[d].w.y, ring[d].w.z, ring[d].w.w};
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const f32x4 v = block_dot<BF16>(xa[d][b], dq(w[b]), C[d][b]);
#pragma unroll
                        for (int r = 0; r < R; ++r)
                            bv[d][b][r] = v[r];
                    }
                }
            }
        };
        auto stage_values = [&](int d) {
            if constexpr (SLOTS) {
                gemv_block_values_slots<BF16>(ring[d].w, ring[d].xa[0], dq, bv[d]);
                return;
            }
            if constexpr (SLOTS2) {
                gemv_block_values_slots2<BF16>(ring[d].w, ring[d].xa[0], ring[d].xa[1], dq, bv[d]);
                return;
            }
            gemv_block_values<BF16, R>(ring[d], ring[d].xa, dq, bv[d]);
        };
        // (a run one stage short of the ring computes the spare stage on
        // zeros rather than branch around it: no branch splits the stages'
        // instructions, q_proj 4.73 -> 4.60 us)
        if constexpr (XF == 2) {
            if (total >= D - 1)
                ahead(std::false_type{});
            else
                ahead(std::true_type{});
        } else if (total >= D - 1) {
#pragma unroll
            for (int d = 0; d < D; ++d)
                stage_values(d);
        } else {
#pragma unroll
            for (int d = 0; d < D; ++d)
                if (d < total)
                    stage_values(d);
        }
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (d < total) {
                const int nq = SHORT ? min(4, plan.nb - 4 * qc) : 4;
                const uint32_t h[4] = {ring[d].s.x & 0xFFFFu, ring[d].s.x >> 16, ring[d].s.y & 0xFFFFu,
                                       ring[d].s.y >> 16};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (!SHORT || i < nq) {
                        const float sc = half_bits_to_float(h[i]);
#pragma unroll
                        for (int r = 0; r < R; ++r)
                            p[r] = __builtin_fmaf(sc, bv[d][i][r], p[r]);
                    }
                }
                finish_quad(qc + 1 == q1 ? q0 : qc + 1);
            }
        }
    }
    for (int base = 0; base < (whole ? 0 : total); base += D) {
        if constexpr (SG) {  // the round's group; all four stages' scales at once
            sg_cur = sg_next;
            issue_fence();
            sg_next = load_group();
            issue_fence();
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int src = (16 * d + c) << 2;
                ring[d].s.x = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)sg_cur.x);
                ring[d].s.y = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)sg_cur.y);
            }
        }
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int ii = base + d;
            if (ii < total) {
                const int qn = qc + 1 == q1 ? q0 : qc + 1;
                if constexpr (XL) {
                    if constexpr (SLOTS)
                        xb[(d + 1) & 1][0] = *(const u32x4 *)(xslot + 256u * (uint32_t)qn);
                    else
                        gemv_x_lds(xb[(d + 1) & 1], xrow, qn);
                }
                if constexpr (SLOTS) {
                    gemv_quad_slots<BF16, SHORT>(ring[d].w, ring[d].s, XL ? xb[d & 1][0] : ring[d].xa[0],
                                                 SHORT ? min(4, plan.nb - 4 * qc) : 4, dq, p);
                } else if constexpr (SLOTS2) {
                    gemv_quad_slots2<BF16, SHORT>(ring[d].w, ring[d].s, ring[d].xa[0], ring[d].xa[1],
                                                  SHORT ? min(4, plan.nb - 4 * qc) : 4, dq, p);
                } else {
                    gemv_quad<BF16, R, SHORT>(ring[d], XL ? xb[d & 1] : ring[d].xa,
                                              SHORT ? min(4, plan.nb - 4 * qc) : 4, dq, p);
                }
                finish_quad(qn);
            }
            // refill D quads ahead.  The scheduling barrier keeps the refill
            // after the stage's use: hoisted above it, the refill's wait (the
            // memory counter retires in order) would drain the whole ring.
            // Refills past the stream's end fall outside the resources'
            // ranges: they return zero without a memory access, so the
            // wave's end does not wait one more round trip for them.
            issue_fence();
            gemv_load<XM, R, !SG>(ring[d], in, left > 0 ? 256u * ql : x_bytes);
            ql = ql + 1 == q1 ? q0 : ql + 1;
            --left;
            issue_fence();
        }
    }

    if constexpr (!SPLIT) {  // y = root for the stream's tiles
        for (int k = 0; k < ntiles; ++k) {
            const int n = 16 * (t0 + k) + c;
            if (n >= N)
                break;
            const float *o = ystage + ((wave * tps + k) * 16 + g) * 16 + c;
            float *yo = y + (size_t)(m0 + g) * N + n;
#pragma unroll
            for (int r = 0; r < R; ++r)
                if (4 * r + g < mrows)
                    yo[4 * r * (size_t)N] = o[64 * r];
        }
    }
    if constexpr (SPLIT) {
        const int W = 1 << log2W;
        const int TW = (blockDim.x >> 6) >> log2W;
        float *rw = red + wave * 16 * 17;
#pragma unroll
        for (int r = 0; r < R; ++r)
            rw[(4 * r + g) * 17 + c] = root[r];
        __syncthreads();
        for (int o = threadIdx.x; o < TW * 256; o += blockDim.x) {
            const int slot = o >> 8, row = (o >> 4) & 15, col = o & 15;
            const int n = 16 * (wgx * TW + slot) + col;
            if (row < mrows && n < N) {
                float v[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    v[j] = j < W ? red[(((slot << log2W) + j) * 16 + row) * 17 + col] : 0.f;
                y[(size_t)(m0 + row) * N + n] = tree_sum<8>(v, W);
            }
        }
    }
}

// ============================================================ GEMV (seg)
// The segment-stationary matrix-vector kernel, for S = 16 segments of at
// most LQ quads (2048 <= K <= 6144).  A workgroup of 16 waves owns `tpw`
// consecutive column tiles; wave j owns segment j of every one of them.  Its
// A operands (x's blocks of segment j) and nothing else of x are loaded once
// into registers, so the workgroup reads x exactly once; the wave then
// streams its segment's tile-quads of all its tiles through a D-deep ring
// (codes and scales only).  Per tile the segment partials go to LDS; every
// TC tiles the workgroup meets at a barrier that does not wait for the ring
// and runs the pairwise tree over the 16 partials; y is written at the end
// (a store inside the streaming loop would make every ring wait drain), by
// the combine itself when it is the only one (measured: gate 10.5 -> 10.3 us
// at one row, 10.75 -> 10.55 at eight).
//
// Ring positions are (tile i, quad q), q in [0, LQ); quads past the
// segment's length are placeholders: their loads fall outside the
// resources' ranges (zero, no memory access) and they compute nothing.
// With one combine (tpw <= TC) the combine writes y directly.
//
// Memory instructions, not bytes, set much of the cost here (measured on
// MI355X, gate at one row: a scale load per stage costs ~0.7 us even when it
// hits the cache), so two inputs are fetched in few of them:
//  * up to four rows (R = 1) the workgroup stages x in LDS, one 16-byte load
//    a thread and 16 KB (waves past x's bytes issue none), and each wave
//    reads its A operands from there (lanes of row slots past the batch read
//    nothing) (gate at one row 10.1 -> 9.7 us, gate|up 17.6 -> 16.6 us);
//    from 5 to 8 rows with segments of up to 2 quads each wave loads its
//    segment's rows in row order, every lane 16 useful bytes, and forms its
//    A operands through its own LDS slot (gate at 5 rows 10.3 -> 9.8 us,
//    gate|up 17.4 -> 16.7 us); otherwise each wave loads them directly,
//    four 16-byte loads a quad;
//  * with rings of four or two stages (LQ <= 2, R <= 2) the scales come in
//    groups of one ring round's positions, one 8-byte load a lane for the
//    group: the lanes of row g load position g's column scales and each
//    position's reach every row by ds_bpermute (four stages: gate 10.1 ->
//    9.9 us, gate|up 17.6 -> 16.8 us, both together 10.1 -> 9.4 us at one
//    to four rows; two stages: gate 8.92 -> 8.77 us at one row).
// grid = (sum over the matrices of ceil(tiles / tpw), ceil(M / 16)),
// block = 1024; a workgroup's matrix is the one whose range of workgroup
// ids holds it (see MatrixItems).  With MR =
// min(M, 16), dynamic LDS: roots [NB][TC][16 seg][MR][16] floats (NB = 1
// if tpw <= TC: one combine after the last tile; else 2, double-buffered),
// then outputs [tpw][MR][16] floats, then (R = 1) x, M rows of 2 K bytes
// and 256 bytes of slack, or (R = 2, LQ <= 2) 16 per-wave slots of 8 rows of
// 256 LQ + 16 bytes (seg_lds_bytes).
// TC: tiles per combine.  Measured on MI355X: with up to 8 tiles per
// workgroup one combine at the end is fastest (gate at one row 10.7 ->
// 10.4 us, at 9 rows 13.2 -> 12.4 us); with more tiles (gate|up, the LM
// head) combining every 2 tiles is, and above 8 rows every tile (the
// partials take 4 KB a row).
__host__ __device__ inline int seg_tc(int M, int tpw) { return tpw <= 8 ? 8 : M > 8 ? 1 : 2; }
__host__ __device__ inline int seg_nbuf(int tc, int tpw) { return tpw <= tc ? 1 : 2; }
// Ring depth of the segment form (a multiple of LQ).  Measured on MI355X:
// 4 stages beat 6, 8 and 10 (a deep per-wave prefetch delays the data each
// wave needs first and scatters the workgroup's accesses).  With 2-quad
// segments, up to 8 tiles a workgroup (one combine) and up to 8 rows, 2
// stages beat 4: 16 waves of a compute unit then keep ~36 KB in flight
// instead of ~72 KB (gate_proj 18944 x 3584 at one row 9.29 -> 8.98 us, at
// eight 9.87 -> 9.54 us; 32768 x 3584 14.4 -> 14.1 us), not from 9 rows on
// (32768 x 3584 at 16 rows 18.1 -> 18.2 us) nor with more tiles.
template <int R, int LQ, int TC>
constexpr int seg_depth()
{
    return LQ == 3 ? 6 : LQ == 2 && TC == 8 && R <= 2 ? 2 : 4;
}

__device__ __forceinline__ void workgroup_barrier_lds()
{
    // LDS writes done, then the barrier; outstanding global loads keep going
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}


template <bool BF16, int R, int LQ, bool SHORT, int TC, int NM>
__global__ __launch_bounds__(1024) void q4_gemv_seg(const uint16_t *__restrict__ x, MatrixItems<NM> items, int M, int K,
                                                    Plan plan, int tpw)
{
    constexpr int D = seg_depth<R, LQ, TC>();  // ring depth: a multiple of LQ
    static_assert(D % LQ == 0, "ring positions must map to fixed quads");
    extern __shared__ __attribute__((aligned(16))) float seg_lds[];
    const int MR = min(M, 16);
    float *roots = seg_lds;                                         // [NB][TC][16 seg][MR][16]
    float *ystage = seg_lds + seg_nbuf(TC, tpw) * TC * 16 * MR * 16;  // [tpw][MR][16]
    uint8_t *x_lds = (uint8_t *)(ystage + tpw * MR * 16);              // x staged or the x slots

    const MatrixSel sel = select_matrix(items);
    const uint8_t *__restrict__ wq = sel.wq;
    const uint16_t *__restrict__ scales = sel.scales;
    float *__restrict__ y = sel.y;
    const int N = sel.N, wg0 = sel.wg0;

    const int lane = threadIdx.x & 63;
    const int j = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // segment
    const int g = lane >> 4, c = lane & 15;
    const int n16 = (N + 15) / 16;
    const int G = plan.G;
    const int m0 = blockIdx.y * 16;
    const int mrows = min(16, M - m0);
    const int t_first = ((int)blockIdx.x - wg0) * tpw;
    const int ntiles = min(tpw, n16 - t_first);
    const int qs = (j * G) >> 4;
    const int len = (((j + 1) * G) >> 4) - qs;  // 1 .. LQ quads

    // this segment's A operands, once: staged through LDS up to four rows,
    // else loaded by the wave
    constexpr bool XLDS = R == 1;
    constexpr int XV = 3;  // 16-byte chunks a thread: 4 rows x 6144 x 2 bytes / 16 KB
    const uint32_t x_bytes = (uint32_t)mrows * (uint32_t)K * 2u;
    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(x + (size_t)m0 * K, x_bytes);
    const int xr = slot_row(c);  // (as in q4_gemv)
    const uint32_t x_lane = xr < mrows ? (uint32_t)xr * (uint32_t)K * 2u + 16u * g : x_bytes;
    const uint32_t x_wave = (uint32_t)(threadIdx.x & ~63u) * 16u;  // the wave's first chunk byte
    u32x4 xs[LQ][4];
    u32x4 xv[XV];
    // 5 to 8 rows, segments of up to 2 quads: the wave loads its segment's
    // rows in row order (every lane 16 useful bytes: 2 LQ loads instead of
    // 4 LQ) and turns them into A operands through its own LDS slot
    constexpr bool XWS = R == 2 && LQ <= 2;
    constexpr uint32_t XS_ROW = 256u * LQ + 16u;  // a row in the slot (padded)
    constexpr int XN = 2 * LQ;                    // 8 rows x 16 LQ chunks / 64 lanes
    u32x4 xw[XN];
    auto xw_chunk = [&](int u, uint32_t &row, uint32_t &ch) {
        const uint32_t id = 64u * (uint32_t)u + (uint32_t)lane;
        row = id / (16u * LQ);
        ch = id % (16u * LQ);
    };
    if constexpr (XWS) {
#pragma unroll
        for (int u = 0; u < XN; ++u) {
            uint32_t row, ch;
            xw_chunk(u, row, ch);
            const uint32_t qq = min((int)(ch >> 4), len - 1);
            const uint32_t off = (int)row < mrows ? row * (uint32_t)K * 2u + 256u * (qs + qq) + 16u * (ch & 15u)
                                                  : x_bytes;
            xw[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
        }
    } else if constexpr (XLDS) {
#pragma unroll
        for (int u = 0; u < XV; ++u)
            if (x_wave + 16384u * u < x_bytes)  // wave-uniform: whole waves past x issue nothing
                xv[u] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, 16u * threadIdx.x + 16384u * u, 0, 0));
    } else {
#pragma unroll
        for (int q = 0; q < LQ; ++q)
#pragma unroll
            for (int b = 0; b < 4; ++b)
                xs[q][b] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                         rx, x_lane + 64u * b + 256u * (qs + min(q, len - 1)), 0, 0));
    }

    // the stream: tiles t_first .. t_first + ntiles - 1, quads qs .. qs + LQ - 1
    const uint32_t tile_b = (uint32_t)G * 1024u, tile_s = (uint32_t)G * 128u;
    const uint32_t w_range = (uint32_t)ntiles * tile_b, s_range = (uint32_t)ntiles * tile_s;
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(wq + (size_t)t_first * G * 1024, w_range);
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(scales + (size_t)t_first * G * 64, s_range);
    const uint32_t w_lane = 16u * lane, s_lane = 8u * c;
    const int npos = ntiles * LQ;
    // up to TC tiles: one combine after the last tile, which stores y itself
    // (no store runs inside the streaming loop); else every TC tiles into
    // the output stage, stored at the end
    const bool one_chunk = tpw <= TC;

    // scale groups (whole ring rounds of D = 4 or 2 stages): the lanes of row
    // g < D load the column scales of position gpos + g (rows g >= D,
    // placeholders and positions past the stream fall outside the range:
    // zero, no memory access).  Measured with the 2-deep ring: gate_proj at
    // one / two rows 8.92 / 9.05 -> 8.77 / 8.87 us against a scale load per
    // stage.
    constexpr bool SG = (D == 4 || D == 2) && LQ <= 2 && R <= 2;
    auto load_group = [&](int gpos) -> u32x2 {
        const int pp = gpos + g;
        const int i = pp / LQ, q = pp % LQ;
        const uint32_t so = g < D && q < len && pp < npos ? (uint32_t)i * tile_s + 128u * (qs + q) : s_range;
        return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, s_lane + so, 0, kWeightLoadPolicy));
    };
    u32x2 sg_cur{0u, 0u}, sg_next{0u, 0u};
    if constexpr (SG) {
        sg_next = load_group(0);
        issue_fence();
    }

    GemvStage ring[D];
    // position -> (tile, quad); live unless the quad is past the segment or
    // the tile past the workgroup's
    auto load = [&](GemvStage &st, int pos, int q) {
        const int i = pos / LQ;  // LQ is a compile-time constant
        const bool live = q < len && pos < npos;
        const uint32_t wo = live ? (uint32_t)i * tile_b + 1024u * (qs + q) : w_range;
        const uint32_t so = live ? (uint32_t)i * tile_s + 128u * (qs + q) : s_range;
        st.w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, w_lane + wo, 0, kWeightLoadPolicy));
        if constexpr (!SG)
            st.s = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, s_lane + so, 0, kWeightLoadPolicy));
    };
#pragma unroll
    for (int d = 0; d < D; ++d) {
        load(ring[d], d, d % LQ);
        issue_fence();
    }
    // (no wait for the whole prefill here: the first stage's wait covers x,
    // loaded before it; measured: gate 10.3 -> 10.1 us)
    if constexpr (XWS) {
        uint8_t *const slot = x_lds + (uint32_t)j * (8u * XS_ROW);
#pragma unroll
        for (int u = 0; u < XN; ++u) {
            uint32_t row, ch;
            xw_chunk(u, row, ch);
            *(u32x4 *)(slot + row * XS_ROW + 16u * ch) = xw[u];
        }
        // (the wave's own slot: its LDS operations complete in order)
#pragma unroll
        for (int q = 0; q < LQ; ++q)
#pragma unroll
            for (int b = 0; b < 4; ++b)
                xs[q][b] = u32x4{0u, 0u, 0u, 0u};
        if (xr < mrows)
#pragma unroll
            for (int q = 0; q < LQ; ++q)
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    xs[q][b] = *(const u32x4 *)(slot + (uint32_t)xr * XS_ROW + 256u * q + 64u * b + 16u * g);
    }
    if constexpr (XLDS) {
#pragma unroll
        for (int u = 0; u < XV; ++u) {
            const uint32_t o = 16u * threadIdx.x + 16384u * u;
            if (x_wave + 16384u * u < x_bytes && o < x_bytes)
                *(u32x4 *)(x_lds + o) = xv[u];
        }
        workgroup_barrier_lds();
        // blocks of a short last quad past the row read the next row or the
        // slack (their block dots are skipped)
        const uint8_t *xrow = x_lds + (uint32_t)xr * (uint32_t)K * 2u + 16u * g;
#pragma unroll
        for (int q = 0; q < LQ; ++q)
#pragma unroll
            for (int b = 0; b < 4; ++b)
                xs[q][b] = u32x4{0u, 0u, 0u, 0u};
        if (xr < mrows)
#pragma unroll
            for (int q = 0; q < LQ; ++q)
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    xs[q][b] = *(const u32x4 *)(xrow + 64u * b + 256u * (qs + min(q, len - 1)));
    }

    const Dequant<BF16> dq;
    // bf16: the segment's corrections once, for all the wave's tiles, where
    // the registers allow (4 LQ accumulator inputs, 16 LQ a lane)
    constexpr bool HOIST = kCorrected<BF16> && LQ <= 2 && R <= 2;
    f32x4 Ch[HOIST ? LQ : 1][4];
    if constexpr (HOIST) {
#pragma unroll
        for (int q = 0; q < LQ; ++q)
#pragma unroll
            for (int b = 0; b < 4; ++b)
                Ch[q][b] = correction<BF16>(xs[q][b], dq);
    }
    float p[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        p[r] = 0.f;
    // ring position pos (tile pos / LQ, quad d % LQ) from stage d
    auto compute = [&](int d, int pos) {
        const int q = d % LQ;
        const int i = pos / LQ;
        if (q < len) {
            const int nq = SHORT && qs + q == G - 1 ? plan.nb - 4 * (G - 1) : 4;
            GemvStage &st = ring[d];
            if constexpr (SG) {  // position d of the group: its scales from row d
                const int src = (16 * d + c) << 2;
                st.s.x = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)sg_cur.x);
                st.s.y = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)sg_cur.y);
            }
            if constexpr (HOIST)
                gemv_quad_pre<BF16, R, SHORT>(st, xs[q], Ch[HOIST ? q : 0], nq, dq, p);
            else
                gemv_quad<BF16, R, SHORT>(st, xs[q], nq, dq, p);
        }
        if (q == LQ - 1) {  // the tile's segment partial is done
            float *rt = roots + ((((i / TC) & 1) * TC + i % TC) * 16 + j) * (MR * 16);
#pragma unroll
            for (int r = 0; r < R; ++r)
                if (4 * r + g < mrows)
                    rt[(4 * r + g) * 16 + c] = p[r];
#pragma unroll
            for (int r = 0; r < R; ++r)
                p[r] = 0.f;
            if (i % TC == TC - 1 || i == ntiles - 1) {  // chunk done: the tree
                workgroup_barrier_lds();
                const int i0 = i - i % TC;
                const float *rc = roots + ((i / TC) & 1) * TC * 16 * (MR * 16);
                for (int o = threadIdx.x; o < TC * 256; o += blockDim.x) {
                    const int k = o >> 8, row = (o >> 4) & 15, col = o & 15;
                    if (i0 + k <= i && row < mrows) {
                        float v[16];
#pragma unroll
                        for (int sg = 0; sg < 16; ++sg)
                            v[sg] = rc[(k * 16 + sg) * (MR * 16) + row * 16 + col];
                        const float root = tree_sum<16>(v, 16);
                        if (one_chunk) {  // after the last tile: straight to y
                            const int n = 16 * (t_first + k) + col;
                            if (n < N)
                                y[(size_t)(m0 + row) * N + n] = root;
                        } else {
                            ystage[((i0 + k) * MR + row) * 16 + col] = root;
                        }
                    }
                }
            }
        }
    };
    auto refill = [&](int d, int pos) {
        issue_fence();
        load(ring[d], pos + D, d % LQ);  // D positions ahead (D % LQ == 0: same quad)
        issue_fence();
    };
    if constexpr (LQ <= 2 && R <= 2) {
        // Whole rounds of the ring in the loop, the remainder (a multiple of
        // LQ) after it: with a guard on each stage's compute in the loop, the
        // compiler has to allow for a round that skips stages and still
        // loops, and its waits for the ring then drain more of it than the
        // round needs (measured: gate 11.8 -> 11.5 us at M = 1).
        // (scale groups: one per round, the next loaded a round ahead)
        int base = 0;
        for (; base + D <= npos; base += D) {
            if constexpr (SG) {
                sg_cur = sg_next;
                issue_fence();
                sg_next = load_group(base + D);
                issue_fence();
            }
#pragma unroll
            for (int d = 0; d < D; ++d) {
                compute(d, base + d);
                refill(d, base + d);
            }
        }
        if constexpr (SG)
            sg_cur = sg_next;
#pragma unroll
        for (int d = 0; d < D - LQ; ++d)
            if (base + d < npos) {
                compute(d, base + d);
                refill(d, base + d);
            }
    } else {
        // three-quad segments or four accumulators: a second copy of the
        // loop body does not fit the 128 registers of a 1024-thread
        // workgroup (it spills), so the stages' compute is guarded inside
        // the loop (the refills past the end read nothing)
        for (int base = 0; base < npos; base += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                if (base + d < npos)
                    compute(d, base + d);
                refill(d, base + d);
            }
        }
    }
    if (one_chunk)
        return;  // y written by the one combine
    __syncthreads();
    for (int o = threadIdx.x; o < ntiles * 256; o += blockDim.x) {
        const int k = o >> 8, row = (o >> 4) & 15, col = o & 15;
        const int n = 16 * (t_first + k) + col;
        if (row < mrows && n < N)
            y[(size_t)(m0 + row) * N + n] = ystage[(k * MR + row) * 16 + col];
    }
}

// =================================================================== GEMM
// The weight-streaming matrix-matrix kernel.  A workgroup of CT waves
// (CT = blockDim / 64, 4..8) owns an output unit of 16 RT rows (RT = 1, 2) by
// CT column tiles and one K-group; wave w computes column tile w of the unit
// for all RT row tiles.  The wave streams its tile's codes and scales
// through a GW_DW-deep register ring (the matrix-vector kernel's loads;
// refills past the K-group's end fall outside the resources' exact ranges
// and read nothing), so every weight byte a workgroup needs is loaded once,
// by the wave that uses it, with many bytes in flight.  The unit's
// activations, 16 RT rows by 128 k per quad (rows of 256 bytes, granules
// swizzled; see gemm_ws_a_offset), are loaded by the waves in chunks of four
// rows into registers two quads ahead and written to a two-stage LDS ring
// one quad ahead; one barrier per quad publishes a stage.  Per block a wave
// dequantizes its B operand once for its RT row tiles and runs RT block
// dots (bf16: 2 RT, the correction of each row tile and its block dot).
//
// The grid is one-dimensional over (column unit, row unit) and K-groups in y:
// workgroup id -> column unit 8 (id / 8 nru) + id % 8, row unit (id / 8) %
// nru, so the row units of one column unit (which read the same weights) are
// eight ids apart: dispatched together, on the same XCD and its L2.
// weight ring stages (registers).  Measured on MI355X with the x register
// sets below: 4 stages beat 6 at 17-32 rows (q_proj at 17 rows 9.9 -> 9.3
// us, gate 24.4 -> 23.6 us) and match them at 124 (fewer registers: 130
// instead of 148)
constexpr int GW_DW = 4;

// The activation stage holds, per row tile, 16 rows of the quad's 256 bytes
// (4 KB); row c's 16-byte granule j sits at granule j ^ c.  One load
// fills four rows (lane l: row l / 16, granule l % 16 of the LDS row), so
// every request covers whole cache lines; the swizzle keeps the A-operand
// reads (lane (g, c): row c, granule 4 i + g of block i) on 16 distinct bank
// groups.
__device__ __forceinline__ uint32_t gemm_ws_a_offset(int rt, int i, int lane)
{
    const int g = lane >> 4, c = lane & 15;
    return (uint32_t)(rt * 4096 + c * 256 + 16 * ((4 * i + g) ^ c));
}

// One quad of a wave's column tile for its RT row tiles: codes w and
// scales s from the register ring, the A operands from the LDS stage stg.
// Few waves share a SIMD and they leave each barrier together, so at one
// row tile the quad is laid out for latency: every A read first, then every
// B operand, every block dot, and last the scale-accumulates in block order
// (block by block, each block paid an LDS round trip and a matrix-core
// latency in series).  At two row tiles that layout's registers cost more
// occupancy than it saves, and the blocks go one by one.  Either way each
// row's blocks accumulate in ascending order.
template <bool BF16, int RT, bool SHORT>
__device__ __forceinline__ void gemm_ws_quad(u32x4 w, u32x2 s, const uint8_t *stg, int lane, int nq,
                                             const Dequant<BF16> &dq, f32x4 (&p)[RT])
{
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    auto scale = [&](int i) {
        const uint32_t sd = i < 2 ? s.x : s.y;
        return half_bits_to_float((i & 1) ? sd >> 16 : sd & 0xFFFFu);
    };
    if constexpr (RT == 1) {
        u32x4 A[4], B[4];
        f32x4 C[4], Dm[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            A[i] = *(const u32x4 *)(stg + gemm_ws_a_offset(0, i, lane));
#pragma unroll
        for (int i = 0; i < 4; ++i)
            B[i] = dq(wd[i]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            C[i] = correction<BF16>(A[i], dq);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            Dm[i] = block_dot<BF16>(A[i], B[i], C[i]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (!SHORT || i < nq)  // blocks past a short last quad: not accumulated
                scale_accumulate(p[0], scale(i), Dm[i]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (!SHORT || i < nq) {
                const u32x4 B = dq(wd[i]);
                u32x4 A[RT];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    A[rt] = *(const u32x4 *)(stg + gemm_ws_a_offset(rt, i, lane));
                // the block dots first, so they overlap in the matrix pipe
                f32x4 C[RT], Dm[RT];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    C[rt] = correction<BF16>(A[rt], dq);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    Dm[rt] = block_dot<BF16>(A[rt], B, C[rt]);
                const float dsc = scale(i);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    scale_accumulate(p[rt], dsc, Dm[rt]);
            }
        }
    }
}

template <bool BF16, int RT, bool SHORT>
__global__ __launch_bounds__(512) void q4_gemm_ws(const uint16_t *__restrict__ x, const uint8_t *__restrict__ wq,
                                                  const uint16_t *__restrict__ scales, float *__restrict__ out,
                                                  int M, int N, int K, Plan plan, int Gk, int ncu, int nru,
                                                  int write_partial)
{
    constexpr int NCH = 4 * RT;  // x chunks per stage
    constexpr int XSTAGE = NCH * 1024;
    __shared__ __attribute__((aligned(1024))) uint8_t xring[2 * XSTAGE];

    const int CT = __builtin_amdgcn_readfirstlane((int)(blockDim.x >> 6));
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, c = lane & 15;
    const int id = blockIdx.x;
    const int cu = 8 * (id / (8 * nru)) + id % 8;
    const int ru = (id / 8) % nru;
    if (cu >= ncu)
        return;  // the whole workgroup, before any barrier
    const int m0 = ru * 16 * RT;
    const int mrows = __builtin_amdgcn_readfirstlane(min(16 * RT, M - m0));
    const int G = plan.G;
    const int n16 = (N + 15) / 16;
    const int ct = cu * CT + w;  // the wave's column tile
    const bool live_ct = ct < n16;
    // K-group: segments [j0, j0 + L), quads [qbeg, qend)
    const int L = plan.S / Gk;
    const int j0 = blockIdx.y * L;
    const int qbeg = (j0 * G) >> plan.log2S;
    const int qend = ((j0 + L) * G) >> plan.log2S;
    const int nquads = qend - qbeg;

    // x rows m0 .. m0 + mrows - 1 (rows past them: offsets past the range)
    const uint32_t xrow = 2u * (uint32_t)K;
    const uint32_t x_range = __builtin_amdgcn_readfirstlane(mrows * (int)xrow);
    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(x + (size_t)m0 * K, x_range);
    // the wave's tile, quads qbeg .. qend - 1 (a spare wave: empty ranges)
    const size_t tq = (size_t)min(ct, n16 - 1) * G + qbeg;
    const uint32_t w_range = __builtin_amdgcn_readfirstlane(live_ct ? nquads * 1024 : 0);
    const uint32_t s_range = __builtin_amdgcn_readfirstlane(live_ct ? nquads * 128 : 0);
    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(wq + tq * 1024, w_range);
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(scales + tq * 64, s_range);

    // x of quad qq: the wave's chunks (RT of them: chunk w + CT h, four rows
    // each) into registers, then into LDS stage qq % 2 (lane l's 16 bytes at
    // 16 l of the chunk).  Chunks past the quads fall outside x's range (zero,
    // no memory access).
    const int xr = lane >> 4, xj = lane & 15;  // row in the chunk, LDS granule
    // x register sets: x is loaded XSETS - 1 quads ahead of its use
    constexpr int XSETS = RT == 1 ? 4 : 2;  // a divisor of GW_DW; more at two row tiles cost occupancy
    u32x4 xreg[XSETS][RT];
    auto load_x = [&](u32x4 (&xv)[RT], int qq) {
        const bool live = qq < nquads;
        const int q = qbeg + qq;
#pragma unroll
        for (int h = 0; h < RT; ++h) {
            const int ch = w + CT * h;  // chunk = row tile * 4 + group of four rows
            if (ch < NCH) {
                const int row = 16 * (ch >> 2) + 4 * (ch & 3) + xr;  // in the unit
                const uint32_t off =
                    live ? (uint32_t)row * xrow + 256u * q + 16u * (uint32_t)(xj ^ (row & 15)) : x_range;
                xv[h] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
            }
        }
    };
    auto write_x = [&](const u32x4 (&xv)[RT], int qq) {
        uint8_t *stg = xring + (qq & 1) * XSTAGE;
#pragma unroll
        for (int h = 0; h < RT; ++h) {
            const int ch = w + CT * h;
            if (ch < NCH)
                *(u32x4 *)(stg + ch * 1024 + 16 * lane) = xv[h];
        }
    };
    struct WStage {
        u32x4 w;
        u32x2 s;
    };
    WStage ring[GW_DW];
    uint32_t w_off = 0, s_off = 0;
    auto issue_w = [&](WStage &st) {
        st.w = __builtin_bit_cast(u32x4,
                                  __builtin_amdgcn_raw_buffer_load_b128(rw, 16u * lane + w_off, 0, kWeightLoadPolicy));
        st.s = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, 8u * c + s_off, 0, kWeightLoadPolicy));
        w_off += 1024u;
        s_off += 128u;
    };

    // x of quad t goes out at quad t - XSETS into register set t % XSETS and
    // into LDS at quad t - 1; the barrier that opens quad t publishes it.
    // Loaded several quads before its write, the wait the compiler puts
    // before the write (it counts conservatively) covers only old loads, so
    // the weight ring keeps its depth (loaded one quad before, the write
    // waited for the previous quad's weight refill).  The
    // weight stages are ordinary register loads the compiler waits for.  No
    // direct global-to-LDS loads: mixed with register loads on the one
    // memory counter, an immediate wait did not reliably cover them (stale
    // activation chunks, measured), and here nothing relies on which loads a
    // count covers.
    static_assert(GW_DW % XSETS == 0 && GW_DW % 2 == 0, "register sets and LDS stages by static index");
#pragma unroll
    for (int k = 0; k < XSETS; ++k)
        load_x(xreg[k], k);
    issue_fence();
#pragma unroll
    for (int d = 0; d < GW_DW; ++d) {
        issue_w(ring[d]);
        issue_fence();
    }
    write_x(xreg[0], 0);
    // Everything the prologue issued lands before the loop (it went out
    // together, and the first quad needs its first loads): with loads still
    // pending from the prologue, the loop header merges two different
    // histories and the compiler's waits for the weight stages collapse to
    // "almost everything landed", a memory round trip per quad.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    const Dequant<BF16> dq;
    f32x4 p[RT];
    TreeStack<RT, f32x4> stack;
#pragma unroll
    for (int a = 0; a < RT; ++a)
        p[a] = (f32x4){0.f, 0.f, 0.f, 0.f};
    int li = 0;
    int seg_end = ((j0 + 1) * G) >> plan.log2S;

    // One quad: stage d of the weight ring, quad qq of the K-group.
    auto quad = [&](int d, int qq) {
        workgroup_barrier_lds();  // stage qq written, stage qq + 1 free
        load_x(xreg[d % XSETS], qq + XSETS);
        issue_fence();

        const uint8_t *stg = xring + (qq & 1) * XSTAGE;
        const int q = qbeg + qq;
        // blocks in the quad: 4, except a short last quad (SHORT only)
        const int nq = SHORT ? min(4, plan.nb - 4 * q) : 4;
        if (live_ct)
            gemm_ws_quad<BF16, RT, SHORT>(ring[d].w, ring[d].s, stg, lane, nq, dq, p);
        if (q + 1 == seg_end) {  // segment j0 + li done
            if (!stack.push_branch(p, li, L)) {
#pragma unroll
                for (int a = 0; a < RT; ++a)
                    p[a] = (f32x4){0.f, 0.f, 0.f, 0.f};
            }
            ++li;
            seg_end = ((j0 + li + 1) * G) >> plan.log2S;
        }
        write_x(xreg[(d + 1) % XSETS], qq + 1);
        issue_fence();
        issue_w(ring[d]);  // quad qq + GW_DW (past the end: reads nothing)
        issue_fence();
    };
    // Whole rounds of the ring in the loop, the remainder after it: with a
    // guard on each stage inside the loop, the compiler has to allow for a
    // round that skips stages and still loops, and its waits for the weight
    // stages then drain almost every load in flight.
    int base = 0;
    for (; base + GW_DW <= nquads; base += GW_DW) {
#pragma unroll
        for (int d = 0; d < GW_DW; ++d)
            quad(d, base + d);
    }
#pragma unroll
    for (int d = 0; d < GW_DW - 1; ++d)
        if (base + d < nquads)
            quad(d, base + d);
    // the refills past the end (they read nothing) land before the wave ends
    __builtin_amdgcn_s_waitcnt(0x0F70);

    // p holds the K-group's subtree roots
    const int n = 16 * ct + c;
    if (live_ct && n < N) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = m0 + 16 * rt + 4 * g + e;
                if (m < M) {
                    const float v = e == 0 ? p[rt].x : e == 1 ? p[rt].y : e == 2 ? p[rt].z : p[rt].w;
                    if (write_partial)
                        out[((size_t)blockIdx.y * M + m) * N + n] = v;
                    else
                        out[(size_t)m * N + n] = v;
                }
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
    y[i] = tree_sum<16>(v, Gk);
}

// =============================================================== quantize
// Dense weights -> canonical codes and binary16 scales, one thread per block
// of 32 weights of a row.  The rule (the pages leave the quantizer open):
// d = absmax / 7 rounded once to binary16, nearest with ties to even, and
// q = clamp(round_half_even(w / d), -8, 7) + 8 on the exact quotient; a
// block whose d rounds to zero gets d = 0 and codes 8.  Both roundings are
// taken exactly: a float estimate (within one step of the answer whatever
// the division's accuracy) is corrected by comparisons that are exact in
// fp32 -- 7 x a binary16 midpoint has at most 15 significant bits, and the
// residual w - n d is exactly representable, so fma returns it unrounded.
__device__ __forceinline__ float f16_value(uint32_t bits)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

__device__ __forceinline__ uint32_t f16_bits_rne(float f)
{
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// binary16 bits of absmax / 7, nearest, ties to even (absmax finite, >= 0)
__device__ __forceinline__ uint32_t q4_scale_bits(float absmax)
{
    uint32_t db = f16_bits_rne(absmax / 7.0f);
    if (db < 0x7BFFu) {  // the midpoint above is finite
        const float hi = 0.5f * (f16_value(db) + f16_value(db + 1));
        if (7.0f * hi < absmax || (7.0f * hi == absmax && (db & 1u)))
            ++db;
    }
    if (db > 0u && db < 0x7C00u) {
        const float lo = 0.5f * (f16_value(db - 1) + f16_value(db));
        if (7.0f * lo > absmax || (7.0f * lo == absmax && (db & 1u)))
            --db;
    }
    return db;
}

// code of w for scale d > 0: clamp(round_half_even(w / d), -8, 7) + 8
__device__ __forceinline__ uint32_t q4_code(float w, float d)
{
    float n = __builtin_rintf(w / d);
    const float r = __builtin_fmaf(-n, d, w);  // w - n d, exact
    const float h = 0.5f * d;
    const float ar = __builtin_fabsf(r);
    if (ar > h || (ar == h && ((int)n & 1)))
        n += r > 0.0f ? 1.0f : -1.0f;
    n = __builtin_fminf(__builtin_fmaxf(n, -8.0f), 7.0f);
    return (uint32_t)(int)(n + 8.0f);
}

// KIND: 0 binary16, 1 bfloat16, 2 binary32 input.
template <int KIND>
__global__ __launch_bounds__(256) void q4_quantize_kernel(const void *__restrict__ w, uint8_t *__restrict__ codes,
                                                          uint16_t *__restrict__ scales, size_t blocks)
{
    const size_t blk = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (blk >= blocks)
        return;
    float v[32];
    if constexpr (KIND == 2) {
        // (float vectors: this compiler miscompiles a bit_cast of an integer
        // vector's .y/.z/.w component into a read of component 0)
        const f32x4 *src = (const f32x4 *)((const float *)w + blk * 32);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const f32x4 t = src[j];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[4 * j + e] = t[e];
        }
    } else {
        const u32x4 *src = (const u32x4 *)((const uint16_t *)w + blk * 32);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x4 t = src[j];
            const uint32_t wd[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const uint32_t b = (wd[h] >> (16 * e)) & 0xFFFFu;
                    v[8 * j + 2 * h + e] = KIND == 1 ? __builtin_bit_cast(float, b << 16) : f16_value(b);
                }
            }
        }
    }
    float absmax = 0.0f;
#pragma unroll
    for (int k = 0; k < 32; ++k)
        absmax = __builtin_fmaxf(absmax, __builtin_fabsf(v[k]));
    const uint32_t db = q4_scale_bits(absmax);
    const float d = f16_value(db);
    const bool live = db != 0u && db < 0x7C00u;
    uint32_t out[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            word |= (live ? q4_code(v[4 * j + e], d) : 8u) << (8 * e);
        out[j] = word;
    }
    u32x4 *dst = (u32x4 *)(codes + blk * 32);
    dst[0] = (u32x4){out[0], out[1], out[2], out[3]};
    dst[1] = (u32x4){out[4], out[5], out[6], out[7]};
    scales[blk] = (uint16_t)db;
}

// =================================================================== pack
// One thread per (tile, quad, lane l = 16 g + c): gathers the four words of
// lane l (codes of k = 32 b + 8 g + r, blocks b = 4q..4q+3 of column
// 16t + c, code r at bit 4 (r / 2) + 16 (r % 2)) and, for g == 0, the
// column's four scales.  NIBBLES: the codes come as nibble rows [N][K/2]
// (byte j of row n: k = 2j in bits 0..3, k = 2j + 1 in bits 4..7) instead of
// one code per byte [N][K].
template <bool NIBBLES>
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
            if constexpr (NIBBLES) {
                const uint8_t *src = codes + (size_t)n * (K / 2) + 16 * b + 4 * g;
#pragma unroll
                for (int r = 0; r < 8; ++r)
                    v |= (uint32_t)((src[r / 2] >> (4 * (r % 2))) & 0x0Fu) << (4 * (r / 2) + 16 * (r % 2));
            } else {
                const uint8_t *src = codes + (size_t)n * K + 32 * b + 8 * g;
#pragma unroll
                for (int r = 0; r < 8; ++r)
                    v |= (uint32_t)(src[r] & 0x0Fu) << (4 * (r / 2) + 16 * (r % 2));
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
// Launch shape of the GEMV; none of it changes the bits.  Wide N: one
// stream per wave over all of K, `tps` tiles per stream.  Narrow N: one
// workgroup per column tile, W = S / L waves over runs of L segments.  The
// shape depends on (M, N, K) only.

struct GemvShape {
    bool split;
    int xm;  // XM_RING, XM_LDS or XM_SLOT
    int L, tps, D, tw;  // tw: column tiles per split workgroup
    size_t lds;  // dynamic LDS bytes
};

// x is staged in LDS when the rows (and the tile roots) fit in this budget
// (bytes of dynamic LDS per workgroup).
// Dynamic LDS of the split form: what its 8.5 KB of static LDS leaves of the
// 160 KB of a compute unit, less 1 KB (the launcher raises the 64 KB
// default).  Staged x for 4 rows of K = 18944 fits.
constexpr size_t GEMV_XLDS_MAX = 160 * 1024 - 8 * 16 * 17 * 4 - 1024;

static GemvShape gemv_shape(int M, int N, const Plan &plan, int K)
{
    GemvShape sh;
    const int tiles = (N + 15) / 16;
    // Measured on MI355X (7B and 0.5B shapes, M = 1..8): very wide N streams
    // one tile per wave over all of K; otherwise a column tile is split over
    // runs of segments of about 4 quads up to 8 rows or for K <= 1024
    // (k_proj 4.3 -> 4.1 us at one row; at 8 rows k_proj 5.04 -> 4.82 us and
    // q_proj 5.48 -> 5.35 us against runs of 7), else 7; 14 for wide N at one
    // or two rows; one segment for K < 1024 (below).
    sh.split = tiles < 4096;
    int L = 1;
    const int target = (tiles >= 1024 && M <= 2) ? 14 : (M <= 8 || plan.G <= 8) ? 4 : 7;  // quads per run
    while (L < plan.S && ((2 * L * plan.G) >> plan.log2S) <= target)
        L *= 2;
    while (plan.S / L > 8)
        L *= 2;
    // 257..512 tiles with 2048 < K <= 6144 (where the split form takes over
    // from the segment form): four runs a tile, so smaller workgroups share
    // the compute units more evenly (measured: 4608 x 3584 at one row 6.5 ->
    // 6.0 us, 6144 x 4864 8.2 -> 6.9 us)
    if (tiles > 256 && tiles <= 512 && plan.G > 16 && plan.G <= 48)
        L = plan.S / 4;
    // K < 1024 (at most 4 segments of under 2 quads): one segment a run up
    // to 256 tiles, and up to 512 tiles at up to 4 rows (measured: 896 x 896
    // at one row 3.46 -> 3.21 us, 512 x 512 3.52 -> 3.06 us, 4864 x 896 4.18
    // -> 4.05 us; not from 8 rows on at 304 tiles and more, not for the
    // 680-tile grouped 0.5B layer, nor at K = 1024)
    if (plan.S <= 4 && (tiles <= 256 || (M <= 4 && tiles <= 512)))
        L = 1;
    sh.L = L;
    sh.tps = (tiles + 2047) / 2048;  // about 2048 streams
    sh.D = 8;
    sh.tps = sh.tps < GEMV_TPS_MAX ? sh.tps : GEMV_TPS_MAX;
    if (!sh.split)
        sh.L = plan.S;  // one run of all S segments
    // a stream's byte offsets stay below 2^31
    const long long tile_bytes = (long long)plan.G * 1024;
    while (sh.tps > 1 && sh.tps * tile_bytes >= (1LL << 31))
        --sh.tps;
    const size_t rows = (size_t)(M < 16 ? M : 16);
    const size_t xbytes = rows * gemv_xrow_bytes(K) + 256;
    const size_t roots = sh.split ? 0 : (size_t)4 * sh.tps * 256 * sizeof(float);
    const bool fits = roots + xbytes <= GEMV_XLDS_MAX;
    // Measured on MI355X, weights streaming from HBM.  Split form up to 8
    // rows: x loaded in the slot layout and used as loaded
    // (gemv_quad_slots / gemv_quad_slots2: 5 or 6 MFMAs a quad, no gathering
    // of x), except at one row with eight runs a tile and K >= 8192, where x
    // is staged once per workgroup and read in the same layout, so the loop
    // issues no x loads.  Against x through per-wave LDS slots: q_proj at 1 /
    // 4 / 5 / 8 rows 4.34 / 4.40 / 4.72 / 4.90 -> 4.11 / 4.23 / 4.45 / 4.74
    // us, k_proj 3.77 / 3.98 / 4.25 / 4.47 -> 3.57 / 3.80 / 4.04 / 4.36 us,
    // down_proj at 2 / 4 / 5 rows 10.22 / 10.58 / 11.6 -> 9.34 / 10.21 /
    // 11.2 us (8 rows: 12.6 either way); staged at one row: down_proj 9.70
    // -> 9.30 us (at 2 and 4 rows staging costs more than it saves).  One
    // stream per wave (very wide N): x staged up to 4 rows, else in the ring.
    sh.xm = fits && M <= 4 ? XM_LDS : XM_RING;
    if (sh.split && M <= 8)
        sh.xm = M == 1 && plan.S / sh.L == 8 && plan.G >= 64 && fits ? XM_LDS : XM_SLOT;
    sh.tw = 1;  // larger workgroups sharing one copy of x measured slower
    if (sh.xm != XM_LDS && sh.split)
        sh.D = 4;  // x rides in the ring: up to 22 registers a stage
    sh.lds = roots + (sh.xm == XM_LDS ? xbytes : 0);
    return sh;
}

struct GemvArgs {
    dim3 grid, block;
    size_t lds;
    hipStream_t stream;
    const uint16_t *x;
    int M, K, L, tps;
    Plan plan;
    MatrixItems<kGroupMax> items;  // the matrices and their workgroup ranges
};

// The kernels' item block for `count` matrices, matrix i taking the
// workgroups of ceil(tiles_i / per_wg) (grid x = the return value).
static int fill_items(MatrixItems<kGroupMax> &mi, const GroupItem *items, int count, int per_wg)
{
    mi = MatrixItems<kGroupMax>{};
    mi.count = count;
    int wg = 0;
    for (int i = 0; i < count; ++i) {
        wg += ((items[i].N + 15) / 16 + per_wg - 1) / per_wg;
        mi.wg_end[i] = wg;
        mi.wq[i] = items[i].wq;
        mi.scales[i] = items[i].scales;
        mi.y[i] = items[i].y;
        mi.N[i] = items[i].N;
    }
    return wg;
}

// The first NM entries of the launch's table.
template <int NM>
static MatrixItems<NM> narrow_items(const MatrixItems<kGroupMax> &m)
{
    MatrixItems<NM> r{};
    r.count = m.count;
    for (int i = 0; i < NM; ++i) {
        r.wg_end[i] = m.wg_end[i];
        r.wq[i] = m.wq[i];
        r.scales[i] = m.scales[i];
        r.y[i] = m.y[i];
        r.N[i] = m.N[i];
    }
    return r;
}

// Whether every run of the split form (L segments, S / L runs a tile) has
// at most D quads, so that the prefill holds it whole.
static bool split_runs_whole(const Plan &plan, int L, int D)
{
    for (int seg0 = 0; seg0 < plan.S; seg0 += L)
        if ((((seg0 + L) * plan.G) >> plan.log2S) - ((seg0 * plan.G) >> plan.log2S) > D)
            return false;
    return true;
}

template <bool BF16, int R, int D, bool SPLIT, int XL, int NM>
static void launch_gemv_n(const GemvArgs &a)
{
    if constexpr (XL == XM_LDS) {
        static const bool lds_raised = [] {
            // a failure here leaves the default limit; the launch then reports it
            (void)hipFuncSetAttribute((const void *)q4_gemv<BF16, R, D, true, SPLIT, XL, NM, 0>,
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)GEMV_XLDS_MAX);
            (void)hipFuncSetAttribute((const void *)q4_gemv<BF16, R, D, false, SPLIT, XL, NM, 0>,
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)GEMV_XLDS_MAX);
            return true;
        }();
        (void)lds_raised;
    }
    const MatrixItems<NM> items = narrow_items<NM>(a.items);
    // bf16 split-form runs that the prefill holds whole, up to 8 rows: x
    // first and the corrections ahead of the codes
    if constexpr (BF16 && SPLIT && R <= 2 && XL != XM_LDS) {
        if (split_runs_whole(a.plan, a.L, D)) {
            if (a.plan.nb & 3)
                hipLaunchKernelGGL((q4_gemv<BF16, R, D, true, SPLIT, XL, NM, 2>), a.grid, a.block, a.lds, a.stream,
                                   a.x, items, a.M, a.K, a.plan, a.L, a.tps);
            else
                hipLaunchKernelGGL((q4_gemv<BF16, R, D, false, SPLIT, XL, NM, 2>), a.grid, a.block, a.lds, a.stream,
                                   a.x, items, a.M, a.K, a.plan, a.L, a.tps);
            return;
        }
    }
    // otherwise x first in the prefill at one row (x in the ring)
    if constexpr (R == 1 && XL != XM_LDS) {
        if (a.M == 1) {
            if (a.plan.nb & 3)
                hipLaunchKernelGGL((q4_gemv<BF16, R, D, true, SPLIT, XL, NM, 1>), a.grid, a.block, a.lds, a.stream,
                                   a.x, items, a.M, a.K, a.plan, a.L, a.tps);
            else
                hipLaunchKernelGGL((q4_gemv<BF16, R, D, false, SPLIT, XL, NM, 1>), a.grid, a.block, a.lds, a.stream,
                                   a.x, items, a.M, a.K, a.plan, a.L, a.tps);
            return;
        }
    }
    if (a.plan.nb & 3)
        hipLaunchKernelGGL((q4_gemv<BF16, R, D, true, SPLIT, XL, NM, 0>), a.grid, a.block, a.lds, a.stream, a.x,
                           items, a.M, a.K, a.plan, a.L, a.tps);
    else
        hipLaunchKernelGGL((q4_gemv<BF16, R, D, false, SPLIT, XL, NM, 0>), a.grid, a.block, a.lds, a.stream, a.x,
                           items, a.M, a.K, a.plan, a.L, a.tps);
}

// A group's table only for the split form (the streaming form runs one
// matrix).
template <bool BF16, int R, int D, bool SPLIT, int XL>
static void launch_gemv_v(const GemvArgs &a)
{
    if constexpr (SPLIT) {
        if (a.items.count > 1) {
            launch_gemv_n<BF16, R, D, SPLIT, XL, kGroupMax>(a);
            return;
        }
    }
    launch_gemv_n<BF16, R, D, SPLIT, XL, 1>(a);
}

// Built variants: x in LDS with a 4-deep ring; x in the slot layout (split
// form, up to 8 rows) with a 4-deep ring; x in the ring with a 4-deep
// (split) or 4/8-deep (one stream per wave) ring.
template <bool BF16, int R>
static void launch_gemv_r(const GemvShape &sh, const GemvArgs &a)
{
    if (sh.xm == XM_LDS) {
        constexpr int DX = 4;  // measured: 4 beats 6 and 8 (down_proj, M <= 4)
        if (sh.split)
            launch_gemv_v<BF16, R, DX, true, XM_LDS>(a);
        else
            launch_gemv_v<BF16, R, DX, false, XM_LDS>(a);
        return;
    }
    if constexpr (R <= 2) {
        if (sh.xm == XM_SLOT) {  // (split form only)
            launch_gemv_v<BF16, R, 4, true, XM_SLOT>(a);
            return;
        }
    }
    if (sh.split) {
        launch_gemv_v<BF16, R, 4, true, XM_RING>(a);
    } else if (sh.D == 4) {
        launch_gemv_v<BF16, R, 4, false, XM_RING>(a);
    } else {
        launch_gemv_v<BF16, R, 8, false, XM_RING>(a);
    }
}

template <bool BF16>
static void launch_gemv_b(int R, const GemvShape &sh, const GemvArgs &a)
{
    if (R == 1)
        launch_gemv_r<BF16, 1>(sh, a);
    else if (R == 2)
        launch_gemv_r<BF16, 2>(sh, a);
    else
        launch_gemv_r<BF16, 4>(sh, a);
}

// ---- the segment-stationary form
// The segment-stationary form runs one 1024-thread workgroup per compute
// unit, so it may take LDS beyond the default 64 KB dynamic limit.
constexpr size_t SEG_LDS_MAX = 160 * 1024;

template <bool BF16, int R, int LQ, int TC, int NM>
static void launch_seg_n(const GemvArgs &a)
{
    static const bool lds_raised = [] {
        // a failure here leaves the default limit; the launch then reports it
        (void)hipFuncSetAttribute((const void *)q4_gemv_seg<BF16, R, LQ, true, TC, NM>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)SEG_LDS_MAX);
        (void)hipFuncSetAttribute((const void *)q4_gemv_seg<BF16, R, LQ, false, TC, NM>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)SEG_LDS_MAX);
        return true;
    }();
    (void)lds_raised;
    const MatrixItems<NM> items = narrow_items<NM>(a.items);
    if (a.plan.nb & 3)
        hipLaunchKernelGGL((q4_gemv_seg<BF16, R, LQ, true, TC, NM>), a.grid, a.block, a.lds, a.stream, a.x, items,
                           a.M, a.K, a.plan, a.tps);
    else
        hipLaunchKernelGGL((q4_gemv_seg<BF16, R, LQ, false, TC, NM>), a.grid, a.block, a.lds, a.stream, a.x, items,
                           a.M, a.K, a.plan, a.tps);
}

template <bool BF16, int R, int LQ, int TC>
static void launch_seg_t(const GemvArgs &a)
{
    if (a.items.count > 1)
        launch_seg_n<BF16, R, LQ, TC, kGroupMax>(a);
    else
        launch_seg_n<BF16, R, LQ, TC, 1>(a);
}

template <bool BF16, int R, int LQ>
static void launch_seg_v(const GemvArgs &a)
{
    if constexpr (R == 4) {
        if (seg_tc(a.M, a.tps) == 8)
            return launch_seg_t<BF16, R, LQ, 8>(a);
        if (seg_tc(a.M, a.tps) == 1)
            return launch_seg_t<BF16, R, LQ, 1>(a);
    } else {
        if (seg_tc(a.M, a.tps) == 8)
            return launch_seg_t<BF16, R, LQ, 8>(a);
    }
    launch_seg_t<BF16, R, LQ, 2>(a);
}

template <bool BF16, int R>
static void launch_seg_r(int LQ, const GemvArgs &a)
{
    if (LQ == 1)
        launch_seg_v<BF16, R, 1>(a);
    else if constexpr (R == 4)  // seg_shape: no 3-quad segments at R = 4
        launch_seg_v<BF16, R, 2>(a);
    else if (LQ == 2)
        launch_seg_v<BF16, R, 2>(a);
    else
        launch_seg_v<BF16, R, 3>(a);
}

template <bool BF16>
static void launch_seg_b(int R, int LQ, const GemvArgs &a)
{
    if (R == 1)
        launch_seg_r<BF16, 1>(LQ, a);
    else if (R == 2)
        launch_seg_r<BF16, 2>(LQ, a);
    else
        launch_seg_r<BF16, 4>(LQ, a);
}

// The segment-stationary form applies with S = 16 segments of at most 3
// quads, more than 256 column tiles and its LDS within 160 KB.  tpw: tiles
// per workgroup, about one workgroup per compute unit.
static bool seg_fits_k(int M, const Plan &plan, int &LQ)
{
    if (plan.S != 16)
        return false;
    LQ = (plan.G + 15) / 16;
    // 3-quad segments at R = 4: 128 registers do not hold them
    return !(LQ > 3 || (LQ == 3 && M > 8));
}

static size_t seg_lds_bytes(int M, int K, int tpw)
{
    const int MR = M < 16 ? M : 16;
    const int tc = seg_tc(M, tpw);
    // up to four rows x is staged too (2 K bytes a row and 256 of slack);
    // from 5 to 8 rows with segments of up to 2 quads each wave has a slot of
    // 8 rows of 256 LQ + 16 bytes
    const Plan plan = make_plan(K);
    const int LQ = (plan.G + 15) / 16;
    const size_t x = M <= 4 ? (size_t)M * K * 2 + 256
                     : (M <= 8 && plan.S == 16 && LQ <= 2) ? (size_t)16 * 8 * (256 * LQ + 16) : 0;
    return (size_t)64 * MR * (seg_nbuf(tc, tpw) * tc * 16 + tpw) + x;
}

static bool seg_shape(int M, int N, const Plan &plan, int &LQ, int &tpw, size_t &lds)
{
    if (!seg_fits_k(M, plan, LQ))
        return false;
    const int tiles = (N + 15) / 16;
    // measured on MI355X: with one tile per workgroup or fewer (N <= 4096)
    // the split form is faster; up to 512 tiles also with 3-quad segments
    // (6144 x 4864 at one row 8.8 -> 6.9 us) and with 2-quad segments up to
    // 4 rows (4608 x 3584 6.5 -> 6.0 us), not from 5 rows on (6144 x 3584
    // at 8 rows 7.1 against 7.3 us)
    if (tiles <= 256 || (tiles <= 512 && (LQ == 3 || (LQ == 2 && M <= 4))))
        return false;
    tpw = (tiles + 255) / 256;
    lds = seg_lds_bytes(M, plan.nb * 32, tpw);
    return lds <= SEG_LDS_MAX;
}

// The split or streaming form over the matrices of `items` (all with the
// shape sh); false if sh is the streaming form and there are several.
static bool launch_gemv_items(const void *x, bool bf16, const GroupItem *items, int count, int M, int K,
                              const Plan &plan, const GemvShape &sh, hipStream_t stream)
{
    GemvArgs a;
    if (sh.split) {
        const int W = plan.S / sh.L;
        const int TW = sh.tw;
        a.grid = dim3((unsigned)fill_items(a.items, items, count, TW), (M + 15) / 16);
        a.block = dim3(64 * W * TW);
    } else {
        if (count != 1)
            return false;
        const int streams = ((items[0].N + 15) / 16 + sh.tps - 1) / sh.tps;
        fill_items(a.items, items, 1, 1);
        a.items.wg_end[0] = (streams + 3) / 4;
        a.grid = dim3((unsigned)a.items.wg_end[0], (M + 15) / 16);
        a.block = dim3(256);
    }
    a.lds = sh.lds;
    a.stream = stream;
    a.x = (const uint16_t *)x;
    a.M = M;
    a.K = K;
    a.L = sh.L;
    a.tps = sh.tps;
    a.plan = plan;
    // accumulator rows per lane: ceil(rows / 4), with 3 rounded up to 4
    const int rows = M < 16 ? M : 16;
    const int R = rows <= 4 ? 1 : rows <= 8 ? 2 : 4;
    // every 16-row slice but a last short one has 16 rows
    if (bf16)
        launch_gemv_b<true>(R, sh, a);
    else
        launch_gemv_b<false>(R, sh, a);
    return true;
}

// The segment form over the matrices of `items`, tpw tiles per workgroup.
static void launch_seg_items(const void *x, bool bf16, const GroupItem *items, int count, int M, int K,
                             const Plan &plan, int LQ, int tpw, size_t lds, hipStream_t stream)
{
    GemvArgs a;
    a.grid = dim3((unsigned)fill_items(a.items, items, count, tpw), (unsigned)((M + 15) / 16));
    a.block = dim3(1024);
    a.lds = lds;
    a.stream = stream;
    a.x = (const uint16_t *)x;
    a.M = M;
    a.K = K;
    a.L = 1;
    a.tps = tpw;
    a.plan = plan;
    const int rows = M < 16 ? M : 16;
    const int R = rows <= 4 ? 1 : rows <= 8 ? 2 : 4;
    if (bf16)
        launch_seg_b<true>(R, LQ, a);
    else
        launch_seg_b<false>(R, LQ, a);
}

hipError_t launch_gemv(const void *x, bool bf16, const uint8_t *wq, const uint16_t *scales,
                       float *y, int M, int N, int K, hipStream_t stream)
{
    const Plan plan = make_plan(K);
    const GroupItem item{wq, scales, y, N};
    int LQ, tpw;
    size_t lds;
    if (seg_shape(M, N, plan, LQ, tpw, lds))
        launch_seg_items(x, bf16, &item, 1, M, K, plan, LQ, tpw, lds, stream);
    else
        launch_gemv_items(x, bf16, &item, 1, M, K, plan, gemv_shape(M, N, plan, K), stream);
    return hipGetLastError();
}

bool launch_gemv_grouped(const void *x, bool bf16, const GroupItem *items, int count, int M, int K,
                         hipStream_t stream, hipError_t *err)
{
    if (count < 1 || count > kGroupMax)
        return false;
    const Plan plan = make_plan(K);
    // the group's total width decides the shape, as one matrix that wide
    long long tiles = 0;
    for (int i = 0; i < count; ++i)
        tiles += (items[i].N + 15) / 16;
    int LQ;
    if (seg_fits_k(M, plan, LQ)) {
        // tiles per workgroup from the group's total, about one workgroup
        // per compute unit over all of them; each matrix gets whole
        // workgroups
        const int tpw = (int)((tiles + 255) / 256);
        const size_t lds = seg_lds_bytes(M, K, tpw);
        if (lds <= SEG_LDS_MAX) {
            launch_seg_items(x, bf16, items, count, M, K, plan, LQ, tpw, lds, stream);
            *err = hipGetLastError();
            return true;
        }
    }
    // the split form (a workgroup per column tile of each matrix), unless
    // the group is wide enough for the streaming form: then one call each
    if (tiles >= (1LL << 26))
        return false;
    const GemvShape sh = gemv_shape(M, (int)(16 * tiles), plan, K);
    if (!launch_gemv_items(x, bf16, items, count, M, K, plan, sh, stream))
        return false;
    *err = hipGetLastError();
    return true;
}

static constexpr int kComputeUnits = 256;

// Matrix-matrix shape: row units of 16 RT rows (the rows spread evenly over
// the units), column units of CT tiles (one wave each), K split over Gk
// groups when a workspace allows and the grid would otherwise leave compute
// units idle.  Measured on MI355X (7B shapes, M = 17..124): 16-row units
// beat 32-, 48- and 64-row ones for K <= 8192 up to M = 64, and 32-row units
// win for K = 18944 and for wide N above M = 64 (gate at M = 124: 62.6 ->
// 55.0 us), where sharing each dequantized B operand over two row tiles
// outweighs the occupancy it costs (the row units of a column unit read its
// weights from one L2).
struct GemmWsShape {
    int RT, nru, CT, ncu, gk;
};

static GemmWsShape gemm_ws_shape(int M, int N, int K, size_t workspace_bytes)
{
    const Plan plan = make_plan(K);
    GemmWsShape sh;
    const int tiles = (N + 15) / 16;
    int rt = K > 8192 || (M > 64 && tiles >= 1024) ? 2 : 1;
    // 16 RT rows of x stay below 2^31 bytes (32-bit offsets)
    if ((long long)32 * rt * K >= (1LL << 31))
        rt = 1;  // (K <= 2^25 keeps 16 rows below 2^31 bytes)
    sh.nru = (M + 16 * rt - 1) / (16 * rt);
    const int rows = (M + sh.nru - 1) / sh.nru;
    sh.RT = (rows + 15) / 16;
    // four waves (column tiles) per workgroup: measured faster than eight at
    // M = 17..32 (the barrier holds fewer waves in step) and no slower above
    sh.CT = 4;
    sh.ncu = (tiles + sh.CT - 1) / sh.CT;
    sh.gk = 1;
    while (sh.gk < plan.S && (long long)sh.ncu * sh.nru * sh.gk < kComputeUnits &&
           (size_t)(2 * sh.gk) * M * N * sizeof(float) <= workspace_bytes)
        sh.gk *= 2;
    return sh;
}

size_t gemm_workspace_bytes(int M, int N, int K)
{
    const int gk = gemm_ws_shape(M, N, K, (size_t)-1).gk;
    return gk > 1 ? (size_t)gk * M * N * sizeof(float) : 0;
}

template <bool BF16, int RT>
static void launch_gemm_ws_r(const GemmWsShape &sh, const uint16_t *x, const uint8_t *wq, const uint16_t *scales,
                             float *out, int M, int N, int K, const Plan &plan, hipStream_t stream)
{
    const dim3 grid((unsigned)((sh.ncu + 7) / 8 * 8 * sh.nru), (unsigned)sh.gk);
    const dim3 block((unsigned)(64 * sh.CT));
    const int wp = sh.gk > 1 ? 1 : 0;
    if (plan.nb & 3)
        hipLaunchKernelGGL((q4_gemm_ws<BF16, RT, true>), grid, block, 0, stream, x, wq, scales, out, M, N, K, plan,
                           sh.gk, sh.ncu, sh.nru, wp);
    else
        hipLaunchKernelGGL((q4_gemm_ws<BF16, RT, false>), grid, block, 0, stream, x, wq, scales, out, M, N, K, plan,
                           sh.gk, sh.ncu, sh.nru, wp);
}

template <bool BF16>
static void launch_gemm_ws(const GemmWsShape &sh, const uint16_t *x, const uint8_t *wq, const uint16_t *scales,
                           float *out, int M, int N, int K, const Plan &plan, hipStream_t stream)
{
    if (sh.RT == 1)
        launch_gemm_ws_r<BF16, 1>(sh, x, wq, scales, out, M, N, K, plan, stream);
    else
        launch_gemm_ws_r<BF16, 2>(sh, x, wq, scales, out, M, N, K, plan, stream);
}

hipError_t launch_gemm(const void *x, bool bf16, const uint8_t *wq, const uint16_t *scales,
                       float *y, int M, int N, int K, void *workspace, size_t workspace_bytes,
                       hipStream_t stream)
{
    const Plan plan = make_plan(K);
    const size_t ws = workspace ? workspace_bytes : 0;
    const GemmWsShape sh = gemm_ws_shape(M, N, K, ws);
    const int gk = sh.gk;
    float *out = gk > 1 ? (float *)workspace : y;
    if (bf16)
        launch_gemm_ws<true>(sh, (const uint16_t *)x, wq, scales, out, M, N, K, plan, stream);
    else
        launch_gemm_ws<false>(sh, (const uint16_t *)x, wq, scales, out, M, N, K, plan, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || gk == 1)
        return e;
    const size_t mn = (size_t)M * N;
    hipLaunchKernelGGL(q4_tree_combine, dim3((unsigned)((mn + 255) / 256)), dim3(256), 0, stream,
                       (const float *)workspace, y, mn, gk);
    return hipGetLastError();
}

// ================================================================ scratch
// A fixed device buffer for callers that cannot allocate (code under graph
// capture, tight serving loops): it holds the matrix-matrix kernel's K-split
// partials, which no call needs more than 4 MiB of (the split stops doubling
// once the grid reaches the compute units: fewer than 512 column unit x row
// unit x split workgroups, each unit at most 32 rows by 64 columns, so at
// most 4 x 2048 x 512 bytes).  Each device holds its own copy until the
// process ends; its device address is looked up once per device (the
// array's name is only a host-side stand-in).  Every call on a device shares
// it and leaves the last call's partials in it (each call writes every
// partial it reads, so nothing needs clearing); calls that overlap on one
// device race.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t scratch_buffer(void **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    void *p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with `dev` current
            if (e != hipSuccess)
                return e;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

hipError_t launch_quantize(const void *w, int kind, uint8_t *codes, uint16_t *scales, int N, int K,
                           hipStream_t stream)
{
    const size_t blocks = (size_t)N * (size_t)(K / 32);
    const dim3 grid((unsigned)((blocks + 255) / 256));
    if (kind == 2)
        hipLaunchKernelGGL(q4_quantize_kernel<2>, grid, dim3(256), 0, stream, w, codes, scales, blocks);
    else if (kind == 1)
        hipLaunchKernelGGL(q4_quantize_kernel<1>, grid, dim3(256), 0, stream, w, codes, scales, blocks);
    else
        hipLaunchKernelGGL(q4_quantize_kernel<0>, grid, dim3(256), 0, stream, w, codes, scales, blocks);
    return hipGetLastError();
}

size_t packed_code_bytes(int N, int K) { return (size_t)((N + 15) / 16) * ((K / 32 + 3) / 4) * 1024; }

size_t packed_scale_bytes(int N, int K) { return (size_t)((N + 15) / 16) * ((K / 32 + 3) / 4) * 128; }

hipError_t launch_pack(const uint8_t *codes, bool nibbles, const uint16_t *scales_in, uint8_t *wq,
                       uint16_t *scales_out, int N, int K, hipStream_t stream)
{
    const size_t items = packed_code_bytes(N, K) / 16;
    const dim3 grid((unsigned)((items + 255) / 256));
    if (nibbles)
        hipLaunchKernelGGL(q4_pack_kernel<true>, grid, dim3(256), 0, stream, codes, scales_in, wq, scales_out, N, K,
                           items);
    else
        hipLaunchKernelGGL(q4_pack_kernel<false>, grid, dim3(256), 0, stream, codes, scales_in, wq, scales_out, N,
                           K, items);
    return hipGetLastError();
}

}  // namespace q4
