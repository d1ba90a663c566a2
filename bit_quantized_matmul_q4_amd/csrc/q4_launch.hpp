// q4_launch.hpp -- host-side launchers exported by q4_kernels.hip to the C
// ABI layer (q4_api.cpp).  Arguments are already validated by the caller.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace q4 {

// Multi-row matrix-vector kernel: any M (rows are processed 16 at a time).
hipError_t launch_gemv(const void *x, bool bf16, const uint8_t *wq, const uint16_t *scales,
                       float *y, int M, int N, int K, hipStream_t stream);

// One matrix of a group that shares x, M and K.
struct GroupItem {
    const uint8_t *wq;
    const uint16_t *scales;
    float *y;
    int N;
};

// The group (1..8 matrices) in one launch of the matrix-vector kernel: the
// segment form where it takes K, else the split form.  Returns false,
// launching nothing, for a group whose total width calls for the streaming
// form (then *err is untouched); else the launch status in *err.
bool launch_gemv_grouped(const void *x, bool bf16, const GroupItem *items, int count, int M, int K,
                         hipStream_t stream, hipError_t *err);

// LDS-staged matrix-matrix kernel.  workspace may be NULL (no split of K
// across workgroups); otherwise it holds workspace_bytes bytes.
hipError_t launch_gemm(const void *x, bool bf16, const uint8_t *wq, const uint16_t *scales,
                       float *y, int M, int N, int K, void *workspace, size_t workspace_bytes,
                       hipStream_t stream);

// Bytes of workspace the matrix-matrix kernel can use for this shape.
size_t gemm_workspace_bytes(int M, int N, int K);

// The library's fixed per-device scratch buffer (for the entry point that
// allocates nothing): its size, and its device address on the current device
// (looked up once per device).
constexpr size_t kScratchBytes = size_t(4) << 20;
hipError_t scratch_buffer(void **ptr);

// Canonical codes ([N][K] one per byte, or nibble rows [N][K/2]) and
// scales [N][K/32] -> the tiled layout.
hipError_t launch_pack(const uint8_t *codes, bool nibbles, const uint16_t *scales_in, uint8_t *wq,
                       uint16_t *scales_out, int N, int K, hipStream_t stream);

// Dense weights [N][K] (kind 0 binary16, 1 bfloat16, 2 binary32) ->
// canonical codes [N][K] and binary16 scales [N][K/32].
hipError_t launch_quantize(const void *w, int kind, uint8_t *codes, uint16_t *scales, int N, int K,
                           hipStream_t stream);

// Sizes of the tiled layout.
size_t packed_code_bytes(int N, int K);
size_t packed_scale_bytes(int N, int K);

}  // namespace q4
