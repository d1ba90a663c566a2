/*
 * q4.h -- C ABI of libq4.so, the MI355X (gfx950) library for the 4-bit
 * block-quantized linear layer of LLM decode:
 *
 *     y[M x N] = x[M x K] . dequant(Wq[N x K])^T
 *
 * The operation: "Why Continuous Batching Slowed Down My LLM Inference
 * Engine: A Metal Kernel Investigation", section "Two Rows of Input, Two
 * Different Kernels" -- a 4-bit quantized weight matrix applied to one input
 * row (matrix-vector kernel) or to several rows at once (matrix-matrix
 * kernel), where the rows are token positions of a batching step (section
 * "The Other Request Already Finished").  That page also shows why a row's
 * result must not depend on which kernel ran (sections "Same Prompt,
 * Different Story" and "The Other Request Already Finished"): this library
 * makes every output row bit-identical whatever M is and whichever kernel
 * runs.
 *
 * Weight format (the pages say only "4-bit quantized"; the library fixes):
 *   - blocks of 32 consecutive weights along K; one IEEE binary16 scale d
 *     per block; 4-bit codes q in 0..15; weight value (q - 8) * d (zero and
 *     subnormal scales are legal and used exactly; inf/nan scales are
 *     outside the contract);
 *   - canonical form (input of q4_pack): codes uint8 [N][K] (one code per
 *     byte, bits 0..3), scales binary16 [N][K/32], both row-major;
 *   - packed form (what q4_pack writes and the compute calls read): tiles
 *     of 16 rows (t = n / 16, c = n % 16) by 4 blocks (quad q = b / 4,
 *     i = b % 4), tile order [ceil(N/16)][ceil(K/128)].
 *       Wq: 1024 bytes per tile.  With g in 0..3, the little-endian
 *         32-bit word at byte 16 * (16 g + c) + 4 i holds the codes of
 *         k = 32 b + 8 g + r, r = 0..7, of row n, block b = 4 q + i: code
 *         r at bit 4 (r / 2) + 16 (r % 2) (even r in the low half-word).
 *       Wscales: 64 binary16 per tile; element 4 c + i is d[n][b].
 *     Entries past N rows or K/32 blocks are zero.  The layout makes each
 *     16-byte load of a 64-lane wave contiguous and gives every lane the
 *     codes of its matrix-core operand words, two k per mask-and-or.
 * Activations x: [M][K] row-major, bfloat16 (q4_linear) or binary16
 * (q4_linear_f16).  Output y: float32 [M][N] row-major, overwritten (no
 * bias, no accumulation into y).
 *
 * Pointers passed to the compute calls are DEVICE pointers (memory of the
 * current HIP device).  `stream` is a hipStream_t cast to void* (NULL = the
 * null stream).  Every call only enqueues work on `stream` and returns; it
 * never synchronizes, allocates, frees or retains memory.  The caller owns
 * every buffer.  Aliasing y (or the workspace) with any input is undefined.
 * Calls are thread-safe; the only global state is the crossover threshold.
 *
 * Return value: Q4_OK (0) or a negative status.  Argument checks run before
 * any HIP call, so a failed check launches nothing.  Q4_ERR_HIP keeps the
 * HIP error code, readable through q4_last_hip_error() on the same thread.
 */
#ifndef Q4_H
#define Q4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q4_ABI_VERSION 6

enum q4_status {
    Q4_OK = 0,
    Q4_ERR_NULL = -1,      /* a required pointer is NULL */
    Q4_ERR_SHAPE = -2,     /* M < 1, N < 1, K < 32, K % 32 != 0, K > 2^25, or a size overflows */
    Q4_ERR_ALIGN = -3,     /* a pointer below the alignment its call states */
    Q4_ERR_ENUM = -4,      /* unknown dtype or kernel selector */
    Q4_ERR_HIP = -5,       /* a HIP call failed (see q4_last_hip_error) */
    Q4_ERR_WORKSPACE = -6, /* workspace_bytes non-zero with a NULL workspace */
    Q4_ERR_SCRATCH = -7    /* the call needs more than Q4_SCRATCH_BYTES of scratch */
};

/* Size of the fixed per-device scratch buffer q4_linear_noalloc uses. */
#define Q4_SCRATCH_BYTES (4u << 20)

enum q4_dtype { Q4_F16 = 0, Q4_BF16 = 1, Q4_F32 = 2 /* q4_quantize input only */ };

enum q4_kernel {
    Q4_AUTO = 0, /* the crossover rule (see q4_get_crossover) picks the kernel */
    Q4_GEMV = 1, /* force the multi-row matrix-vector kernel (any M) */
    Q4_GEMM = 2  /* force the LDS-staged matrix-matrix (MFMA tile) kernel */
};

/*
 * y = x . dequant(Wq)^T with bfloat16 activations.
 *   x      bf16  [M][K]          device, 16-byte aligned
 *   Wq     packed codes          device, 16-byte aligned, q4_packed_code_bytes(N, K)
 *   scales packed scales         device, 8-byte aligned, q4_packed_scale_bytes(N, K)
 *   y      fp32  [M][N]          device, 4-byte aligned, overwritten
 * Kernel chosen by the crossover rule (Q4_AUTO), with no workspace.
 * Source: "Why Continuous Batching Slowed Down My LLM Inference Engine: A
 * Metal Kernel Investigation", section "Two Rows of Input, Two Different
 * Kernels" (one quantized weight matrix applied to the batch's rows); the
 * signature and weight format are the task spec's.
 */
int q4_linear(const void *x, const void *Wq, const void *scales, float *y,
              int M, int N, int K, void *stream);

/* Same as q4_linear with binary16 activations (the fp16 workloads: the
 * single matvec and the Qwen2.5-0.5B-shaped set; task spec). */
int q4_linear_f16(const void *x, const void *Wq, const void *scales, float *y,
                  int M, int N, int K, void *stream);

/*
 * Full form.  x_dtype is Q4_BF16 or Q4_F16; kernel is a q4_kernel value.
 * workspace: optional device scratch of workspace_bytes bytes (256-byte
 * aligned) that lets the matrix-matrix kernel split K across workgroups;
 * pass NULL and 0 to run without it (same bits, fewer workgroups).
 * q4_workspace_bytes() gives the size that enables the full split for a
 * shape.  A workspace smaller than that is used for a smaller split.
 * Two calls that share one workspace must not overlap in time.
 * Source: the same page, sections "Two Rows of Input, Two Different Kernels"
 * (matrix-vector vs matrix-matrix kernel) and "Row-by-Row GEMV to the
 * Rescue" (forcing the matrix-vector kernel); the bits do not depend on the
 * kernel (section "Same Prompt, Different Story").
 */
int q4_linear_ex(const void *x, int x_dtype, const void *Wq, const void *scales,
                 float *y, int M, int N, int K, int kernel,
                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * q4_linear_ex without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the call allocates nothing.  Where the
 * matrix-matrix kernel splits K it keeps its partial results in the
 * library's fixed scratch buffer, a static device array of Q4_SCRATCH_BYTES
 * bytes per GPU that lives until the process ends; every need of the current
 * kernels is below that (Q4_ERR_SCRATCH otherwise, before any launch).  The
 * buffer's device address is looked up on the first such call on each
 * device (with that device current).  All calls on one GPU share the buffer
 * and leave their partials in it; two calls that overlap in time on one GPU
 * (other streams, other threads) race and must be serialized by the caller.
 * Same arguments, results and errors as q4_linear_ex otherwise; the bits
 * equal q4_linear_ex's with a workspace.
 */
int q4_linear_noalloc(const void *x, int x_dtype, const void *Wq, const void *scales,
                      float *y, int M, int N, int K, int kernel, void *stream);

/* Workspace bytes that q4_linear_ex can use for this shape and kernel
 * (0 if the kernel uses none).  Pure host computation; 0 for bad shapes.
 * (Library detail; the pages are silent.) */
size_t q4_workspace_bytes(int M, int N, int K, int kernel);

/*
 * Pack the canonical form into the packed form (both described above).
 *   codes    uint8 [N][K]     device, any alignment; only bits 0..3 used
 *   scales   fp16 [N][K/32]   device, 2-byte aligned
 *   Wq       packed codes     device, 16-byte aligned, q4_packed_code_bytes(N, K)
 *   Wscales  packed scales    device, 8-byte aligned, q4_packed_scale_bytes(N, K)
 * K must be a positive multiple of 32.  Bit-exact; padding is written as 0.
 * Source: task spec (the pages say only "4-bit quantized": "Why Continuous
 * Batching Slowed Down My LLM Inference Engine", introduction).
 */
int q4_pack(const uint8_t *codes, const void *scales, uint8_t *Wq, void *Wscales, int N, int K,
            void *stream);

/*
 * q4_pack for codes given as nibble rows, the plain 4-bit row-major form:
 *   Wq_rows  uint8 [N][K/2]   device, any alignment; byte j of row n holds
 *                             k = 2j in bits 0..3 and k = 2j + 1 in bits 4..7
 * Other arguments, results and errors as q4_pack (bit-exact; the same packed
 * bytes as q4_pack of the unpacked codes).
 * Source: task spec (its packed Wq [N x K/2] input format).
 */
int q4_pack_nibbles(const uint8_t *Wq_rows, const void *scales, uint8_t *Wq, void *Wscales, int N, int K,
                    void *stream);

/*
 * Grouped launch: several weight matrices that take the same x (same M, K
 * and activation type), e.g. a layer's q, k and v projections and its gate
 * and up projections, in one dispatch, so the launch and ramp cost of the
 * matrix-vector kernel is paid once for all of them (the per-call dispatch
 * cost "Why Continuous Batching Slowed Down My LLM Inference Engine: A Metal
 * Kernel Investigation", section "Row-by-Row GEMV to the Rescue", blames
 * for the row-by-row scheme's slowdown).
 *   x        [M][K] bf16 or binary16 (x_dtype), device, 16-byte aligned
 *   items    host array of `count` (1..Q4_GROUP_MAX) matrices: packed Wq and
 *            scales of an N_i x K weight (alignment as q4_linear) and y_i
 *            fp32 [M][N_i] (4-byte aligned, overwritten); the y_i must not
 *            overlap each other or any input
 * Every y_i is bit-identical to q4_linear_ex's for that matrix (any kernel):
 * the reduction order depends on K only.  One launch of the matrix-vector
 * kernel when the crossover rule picks it for the group (as q4_linear_ex
 * with Q4_AUTO and this workspace would for each matrix), unless the group
 * is too wide for one launch (65536 columns or more in all where the
 * segment form, 2048 <= K <= 6144, does not take it); else one call per
 * matrix as q4_linear_ex with Q4_AUTO and the given workspace (optional, as
 * for q4_linear_ex; the calls run in stream order, so one workspace of the
 * largest item's q4_workspace_bytes serves them all).  All argument checks
 * (every item's) run before any HIP call.  No allocation.
 */
#define Q4_GROUP_MAX 8
typedef struct q4_group_item {
    const void *Wq;
    const void *scales;
    float *y;
    int N;
} q4_group_item;

int q4_linear_grouped(const void *x, int x_dtype, const q4_group_item *items, int count, int M, int K,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * Quantize dense weights into the canonical form (the input of q4_pack).
 * The pages only call the weights "4-bit quantized"; the rule used, per
 * block of 32 consecutive weights of a row (absmax scaling onto the
 * symmetric codes -7..7 around the offset 8):
 *     d = absmax / 7, rounded once to binary16 (nearest, ties to even);
 *     q = clamp(round_half_even(w / d), -8, 7) + 8, on the exact quotient;
 *     a block whose d rounds to zero gets d = +0 and every code 8.
 * Both roundings are exact, so the result is bit-reproducible anywhere.
 * Source: none on the pages (they never say how the 4-bit codes are made);
 * the plain absmax rule is this library's reading.
 *   w        [N][K] row-major, w_dtype Q4_F32, Q4_BF16 or Q4_F16; device,
 *            16-byte aligned.  Values must be finite with absmax / 7 below
 *            65520 (the binary16 overflow threshold); a block outside that
 *            gets unspecified codes and scale (no error is reported).
 *   codes    uint8 [N][K] (one code 0..15 per byte); device, 16-byte aligned
 *   scales   binary16 [N][K/32]; device, 2-byte aligned
 * K must be a positive multiple of 32.  Enqueues on `stream` like the
 * compute calls; errors as for them (Q4_ERR_ENUM for a bad w_dtype).
 */
int q4_quantize(const void *w, int w_dtype, uint8_t *codes, void *scales, int N, int K, void *stream);

/* Bytes of the packed codes and packed scales of an N x K matrix (0 for a
 * bad shape).  Pure host computation.  (Library layout; pages silent.) */
size_t q4_packed_code_bytes(int N, int K);
size_t q4_packed_scale_bytes(int N, int K);

/* Crossover threshold T: Q4_AUTO uses the matrix-vector kernel iff M <= T,
 * except that for K > 8192 it uses the matrix-matrix kernel already for
 * M > min(T, 8) when the call gets the workspace q4_workspace_bytes(M, N, K,
 * Q4_AUTO) asks for (q4_linear, which has none, then keeps the matrix-vector
 * kernel).  T is initialised from the environment variable Q4_CROSSOVER if
 * set, else the measured default.  q4_set_crossover returns Q4_ERR_SHAPE for
 * T < 0.  The rule never changes results, only speed.
 * Source: "Why Continuous Batching Slowed Down My LLM Inference Engine",
 * sections "Two Rows of Input, Two Different Kernels" (switch at one row)
 * and "Row-by-Row GEMV to the Rescue" (a measured threshold of 4). */
int q4_get_crossover(void);
int q4_set_crossover(int T);

/* Number of K-segments the fixed reduction order uses for this K (1..16),
 * or 0 if K is not a positive multiple of 32.  It depends on K only (the
 * fixed order answers that page's section "Same Prompt, Different Story"). */
int q4_segments(int K);

/* Human-readable text for a status code (static storage).  (Library.) */
const char *q4_strerror(int status);

/* HIP error code of the last Q4_ERR_HIP on the calling thread (0 if none).
 * (Library.) */
int q4_last_hip_error(void);

/* Q4_ABI_VERSION of the loaded library.  (Library.) */
int q4_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* Q4_H */
