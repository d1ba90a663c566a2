// q4_api.cpp -- the C ABI of libq4.so (declared in include/q4.h).
//
// Argument checks, the crossover dispatcher and status codes.  The kernel
// choice follows the row-count switch of "Why Continuous Batching Slowed
// Down My LLM Inference Engine: A Metal Kernel Investigation" (section "Two
// Rows of Input, Two Different Kernels": one row -> matrix-vector, more ->
// matrix-matrix; section "Row-by-Row GEMV to the Rescue": the switch moved to
// a measured threshold, <= 4 rows -> matrix-vector).  Here the threshold is
// the crossover measured on MI355X, and because both kernels share one
// reduction order the choice changes speed only, never the bits.
#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include <hip/hip_runtime_api.h>

#include "../../include/q4.h"
#include "q4_launch.hpp"
#include "q4_plan.hpp"

namespace {

// Measured GEMV -> GEMM crossover on MI355X (rows); M <= T runs the GEMV.
// On the Qwen2.5-7B-shaped layer set (the sum of the six projections' times)
// the matrix-matrix kernel first wins at M = 17, where the matrix-vector
// kernel needs a second 16-row slice (102 vs 106 us); at 16 the matrix-vector
// kernel is 10% faster (73 vs 81 us).  T = 16.
constexpr int kDefaultCrossover = 16;
// Long K (K > 8192), measured: the matrix-vector kernel's time grows with the
// rows (down_proj 3584 x 18944: 16.9 us at 9 rows, 23.2 at 16) while the
// matrix-matrix kernel, split over K, stays near 16 us; from 9 rows on it is
// faster, provided it gets its split workspace (without it, down_proj takes
// several times longer).
constexpr int kLongK = 8192, kLongKCrossover = 8;

thread_local int g_last_hip = 0;

int env_int(const char *name, int fallback)
{
    const char *v = std::getenv(name);
    if (!v || !*v)
        return fallback;
    char *end = nullptr;
    const long r = std::strtol(v, &end, 10);
    if (end == v || *end != '\0' || r < 0 || r > (1 << 30))
        return fallback;
    return (int)r;
}

std::atomic<int> &crossover()
{
    static std::atomic<int> t{env_int("Q4_CROSSOVER", kDefaultCrossover)};
    return t;
}

// Q4_KERNEL=gemv|gemm forces a kernel for Q4_AUTO calls (read once).
int forced_kernel()
{
    static const int k = [] {
        const char *v = std::getenv("Q4_KERNEL");
        if (v && std::strcmp(v, "gemv") == 0)
            return (int)Q4_GEMV;
        if (v && std::strcmp(v, "gemm") == 0)
            return (int)Q4_GEMM;
        return (int)Q4_AUTO;
    }();
    return k;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int check_shape(long long M, long long N, long long K)
{
    if (M < 1 || N < 1 || K < 32 || K % 32 != 0)
        return Q4_ERR_SHAPE;
    // one column tile's packed codes (K / 2 * 16 bytes) and 16 rows of x
    // (32 K bytes) stay below 2^31 bytes: the kernels address them with
    // 32-bit offsets
    if (K > (1LL << 25))
        return Q4_ERR_SHAPE;
    // every element count must fit comfortably in 63 bits and every row
    // index product used by the kernels in size_t
    const long long lim = 1LL << 46;
    if (M > lim / K || N > lim / K || M > lim / N)
        return Q4_ERR_SHAPE;
    return Q4_OK;
}

int hip_status(hipError_t e)
{
    if (e == hipSuccess)
        return Q4_OK;
    g_last_hip = (int)e;
    return Q4_ERR_HIP;
}

}  // namespace

extern "C" {

int q4_abi_version(void) { return Q4_ABI_VERSION; }

int q4_last_hip_error(void) { return g_last_hip; }

const char *q4_strerror(int status)
{
    switch (status) {
    case Q4_OK: return "ok";
    case Q4_ERR_NULL: return "a required pointer is NULL";
    case Q4_ERR_SHAPE: return "bad shape (need M >= 1, N >= 1, K >= 32, K % 32 == 0, sizes in range)";
    case Q4_ERR_ALIGN: return "misaligned pointer (x, Wq, quantizer w and codes: 16 B; packed scales: 8 B; y: 4 B; workspace: 256 B)";
    case Q4_ERR_ENUM: return "unknown dtype or kernel selector";
    case Q4_ERR_HIP: return "HIP launch error (see q4_last_hip_error)";
    case Q4_ERR_WORKSPACE: return "workspace_bytes > 0 with a NULL workspace";
    case Q4_ERR_SCRATCH: return "the call needs more than the library's fixed scratch buffer (Q4_SCRATCH_BYTES)";
    default: return "unknown status";
    }
}

int q4_get_crossover(void) { return crossover().load(std::memory_order_relaxed); }

int q4_set_crossover(int T)
{
    if (T < 0)
        return Q4_ERR_SHAPE;
    crossover().store(T, std::memory_order_relaxed);
    return Q4_OK;
}

int q4_segments(int K)
{
    if (K < 32 || K % 32 != 0)
        return 0;
    return q4::make_plan(K).S;
}

// The kernel Q4_AUTO runs: matrix-vector iff M <= T, except that for
// K > kLongK the matrix-matrix kernel already runs above min(T, 8) rows when
// it has the workspace it asks for (ws_ok).
static int auto_kernel(int M, int K, bool ws_ok)
{
    if (forced_kernel() != Q4_AUTO)
        return forced_kernel();
    const int T = q4_get_crossover();
    if (M > T)
        return Q4_GEMM;
    if (K > kLongK && M > std::min(T, kLongKCrossover) && ws_ok)
        return Q4_GEMM;
    return Q4_GEMV;
}

size_t q4_workspace_bytes(int M, int N, int K, int kernel)
{
    if (check_shape(M, N, K) != Q4_OK)
        return 0;
    const int k = kernel == Q4_AUTO ? auto_kernel(M, K, true) : kernel;
    if (k != Q4_GEMM)
        return 0;
    return q4::gemm_workspace_bytes(M, N, K);
}

// The checks and dispatch shared by q4_linear_ex and q4_linear_noalloc.
// scratch: take the library's fixed device buffer as the workspace (the
// caller passes none).
static int linear_impl(const void *x, int x_dtype, const void *Wq, const void *scales, float *y, int M, int N,
                       int K, int kernel, void *workspace, size_t workspace_bytes, bool scratch, void *stream)
{
    if (!x || !Wq || !scales || !y)
        return Q4_ERR_NULL;
    if (x_dtype != Q4_F16 && x_dtype != Q4_BF16)
        return Q4_ERR_ENUM;
    if (kernel != Q4_AUTO && kernel != Q4_GEMV && kernel != Q4_GEMM)
        return Q4_ERR_ENUM;
    const int sh = check_shape(M, N, K);
    if (sh != Q4_OK)
        return sh;
    if (!aligned(x, 16) || !aligned(Wq, 16) || !aligned(scales, 8) || !aligned(y, 4))
        return Q4_ERR_ALIGN;
    if (workspace_bytes > 0 && !workspace)
        return Q4_ERR_WORKSPACE;
    if (workspace && !aligned(workspace, 256))
        return Q4_ERR_ALIGN;

    const size_t need = q4::gemm_workspace_bytes(M, N, K);
    const int k = kernel == Q4_AUTO
                      ? auto_kernel(M, K, scratch ? need <= q4::kScratchBytes : workspace_bytes >= need)
                      : kernel;
    if (k == Q4_GEMM && scratch) {
        if (need > q4::kScratchBytes)
            return Q4_ERR_SCRATCH;
        if (need > 0) {
            const int st = hip_status(q4::scratch_buffer(&workspace));
            if (st != Q4_OK)
                return st;
            workspace_bytes = need;
        }
    }

    const bool bf16 = x_dtype == Q4_BF16;
    hipStream_t s = (hipStream_t)stream;
    if (k == Q4_GEMV)
        return hip_status(q4::launch_gemv(x, bf16, (const uint8_t *)Wq, (const uint16_t *)scales, y,
                                          M, N, K, s));
    return hip_status(q4::launch_gemm(x, bf16, (const uint8_t *)Wq, (const uint16_t *)scales, y, M, N,
                                      K, workspace_bytes ? workspace : nullptr, workspace_bytes, s));
}

int q4_linear_ex(const void *x, int x_dtype, const void *Wq, const void *scales, float *y,
                 int M, int N, int K, int kernel, void *workspace, size_t workspace_bytes,
                 void *stream)
{
    return linear_impl(x, x_dtype, Wq, scales, y, M, N, K, kernel, workspace, workspace_bytes, false, stream);
}

int q4_linear_noalloc(const void *x, int x_dtype, const void *Wq, const void *scales, float *y, int M, int N,
                      int K, int kernel, void *stream)
{
    return linear_impl(x, x_dtype, Wq, scales, y, M, N, K, kernel, nullptr, 0, true, stream);
}

int q4_linear(const void *x, const void *Wq, const void *scales, float *y, int M, int N, int K,
              void *stream)
{
    return q4_linear_ex(x, Q4_BF16, Wq, scales, y, M, N, K, Q4_AUTO, nullptr, 0, stream);
}

int q4_linear_f16(const void *x, const void *Wq, const void *scales, float *y, int M, int N, int K,
                  void *stream)
{
    return q4_linear_ex(x, Q4_F16, Wq, scales, y, M, N, K, Q4_AUTO, nullptr, 0, stream);
}

size_t q4_packed_code_bytes(int N, int K)
{
    if (check_shape(1, N, K) != Q4_OK)
        return 0;
    return q4::packed_code_bytes(N, K);
}

size_t q4_packed_scale_bytes(int N, int K)
{
    if (check_shape(1, N, K) != Q4_OK)
        return 0;
    return q4::packed_scale_bytes(N, K);
}

int q4_quantize(const void *w, int w_dtype, uint8_t *codes, void *scales, int N, int K, void *stream)
{
    if (!w || !codes || !scales)
        return Q4_ERR_NULL;
    if (w_dtype != Q4_F16 && w_dtype != Q4_BF16 && w_dtype != Q4_F32)
        return Q4_ERR_ENUM;
    const int sh = check_shape(1, N, K);
    if (sh != Q4_OK)
        return sh;
    if (!aligned(w, 16) || !aligned(codes, 16) || !aligned(scales, 2))
        return Q4_ERR_ALIGN;
    const int kind = w_dtype == Q4_F32 ? 2 : w_dtype == Q4_BF16 ? 1 : 0;
    return hip_status(q4::launch_quantize(w, kind, codes, (uint16_t *)scales, N, K, (hipStream_t)stream));
}

static int pack_impl(const uint8_t *codes, bool nibbles, const void *scales, uint8_t *Wq, void *Wscales, int N,
                     int K, void *stream)
{
    if (!codes || !scales || !Wq || !Wscales)
        return Q4_ERR_NULL;
    const int sh = check_shape(1, N, K);
    if (sh != Q4_OK)
        return sh;
    if (!aligned(scales, 2) || !aligned(Wq, 16) || !aligned(Wscales, 8))
        return Q4_ERR_ALIGN;
    return hip_status(q4::launch_pack(codes, nibbles, (const uint16_t *)scales, Wq, (uint16_t *)Wscales, N, K,
                                      (hipStream_t)stream));
}

int q4_pack(const uint8_t *codes, const void *scales, uint8_t *Wq, void *Wscales, int N, int K,
            void *stream)
{
    return pack_impl(codes, false, scales, Wq, Wscales, N, K, stream);
}

int q4_pack_nibbles(const uint8_t *Wq_rows, const void *scales, uint8_t *Wq, void *Wscales, int N, int K,
                    void *stream)
{
    return pack_impl(Wq_rows, true, scales, Wq, Wscales, N, K, stream);
}

int q4_linear_grouped(const void *x, int x_dtype, const q4_group_item *items, int count, int M, int K,
                      void *workspace, size_t workspace_bytes, void *stream)
{
    if (!x || !items)
        return Q4_ERR_NULL;
    if (workspace_bytes > 0 && !workspace)
        return Q4_ERR_WORKSPACE;
    if (workspace && !aligned(workspace, 256))
        return Q4_ERR_ALIGN;
    if (x_dtype != Q4_F16 && x_dtype != Q4_BF16)
        return Q4_ERR_ENUM;
    if (count < 1 || count > Q4_GROUP_MAX)
        return Q4_ERR_SHAPE;
    if (!aligned(x, 16))
        return Q4_ERR_ALIGN;
    q4::GroupItem g[Q4_GROUP_MAX];
    for (int i = 0; i < count; ++i) {
        const q4_group_item &it = items[i];
        if (!it.Wq || !it.scales || !it.y)
            return Q4_ERR_NULL;
        const int sh = check_shape(M, it.N, K);
        if (sh != Q4_OK)
            return sh;
        if (!aligned(it.Wq, 16) || !aligned(it.scales, 8) || !aligned(it.y, 4))
            return Q4_ERR_ALIGN;
        g[i] = q4::GroupItem{(const uint8_t *)it.Wq, (const uint16_t *)it.scales, it.y, it.N};
    }
    const bool bf16 = x_dtype == Q4_BF16;
    hipStream_t s = (hipStream_t)stream;
    // one launch of the matrix-vector kernel where the crossover rule picks
    // it for every matrix (as q4_linear_ex with Q4_AUTO and this workspace
    // would); otherwise, and for groups too wide for one launch, each matrix
    // as q4_linear_ex (the calls are stream-ordered, so they can share the
    // workspace)
    bool ws_ok = workspace != nullptr;
    for (int i = 0; i < count; ++i)
        ws_ok = ws_ok && q4::gemm_workspace_bytes(M, g[i].N, K) <= workspace_bytes;
    if (auto_kernel(M, K, ws_ok) == Q4_GEMV) {
        hipError_t e = hipSuccess;
        if (q4::launch_gemv_grouped(x, bf16, g, count, M, K, s, &e))
            return hip_status(e);
    }
    for (int i = 0; i < count; ++i) {
        const int st = linear_impl(x, x_dtype, g[i].wq, g[i].scales, g[i].y, M, g[i].N, K, Q4_AUTO, workspace,
                                   workspace_bytes, false, stream);
        if (st != Q4_OK)
            return st;
    }
    return Q4_OK;
}

}  // extern "C"
