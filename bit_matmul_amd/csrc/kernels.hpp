// Internal launch interface between the C ABI (api.cpp) and the kernels.
// Callers have validated every argument; these functions only enqueue work. `group`
// is the quantization group along K (32, 64 or 128), K a multiple of 64 and of it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bitmm {

// GEMV / small-M path: y[M, N] = x[M, K] * dequant(w)^T, rows taken 8 at a time.
hipError_t launch_qmv(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
                      const uint16_t* biases, void* y, int64_t M, int64_t N, int64_t K, int bits,
                      int group, bool out_f32, hipStream_t stream);

// Gathered GEMV (MoE decode): output row r reads activation row token_idx[r] (row r if
// token_idx is null) of x[T, K] and expert expert_idx[r] of w[E, N, K*bits/32], any
// order; rows with an out-of-range id are written as zeros.
hipError_t launch_gather_qmv(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
                             const uint16_t* biases, const int32_t* token_idx,
                             const int32_t* expert_idx, void* y, int64_t B, int64_t N, int64_t K,
                             int64_t E, int64_t T, int bits, int group, bool out_f32,
                             hipStream_t stream);

// Matrix-core GEMM for M >= 8.
hipError_t launch_qmm_mfma(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
                           const uint16_t* biases, void* y, int64_t M, int64_t N, int64_t K,
                           int bits, int group, bool out_f32, hipStream_t stream);

// Expert-gathered GEMM: prepare (validation + per-expert offsets into workspace),
// then the grouped matrix-core kernel.
size_t gather_workspace_bytes(int64_t E);
hipError_t launch_gather_qmm(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
                             const uint16_t* biases, const int32_t* expert_idx, void* y,
                             int64_t B, int64_t N, int64_t K, int64_t E, int bits, int group,
                             bool out_f32, void* workspace, hipStream_t stream);

// Indexed GatherQMM (rows in any order, optional token index): a counting sort of the
// rows by expert into the workspace, then the grouped GEMM over the sorted rows.
size_t gather_indexed_workspace_bytes(int64_t B, int64_t E);
int64_t gather_indexed_max_experts();
hipError_t launch_gather_qmm_indexed(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
                                     const uint16_t* biases, const int32_t* token_idx,
                                     const int32_t* expert_idx, void* y, int64_t B, int64_t N,
                                     int64_t K, int64_t E, int64_t T, int bits, int group,
                                     bool out_f32, void* workspace, hipStream_t stream);

}  // namespace bitmm
