// Internal launch interface between the C ABI (api.cpp) and the kernels.
// Callers have validated every argument; these functions only enqueue work. `group`
// is the quantization group along K (32, 64 or 128), K a multiple of 64 and of it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bitmm {

// Output element types of the matrix-core epilogue (bitmm_out's values).
enum OutType { kOutBf16 = 0, kOutF32 = 1, kOutF16 = 2 };

// Kernel-choice record of the calling thread (bitmm_last_launches): each C-ABI call
// starts an empty record, and every launch site appends one line naming the kernel it
// enqueued, with its template arguments, grid, workgroup size and LDS bytes.
void launch_log_begin();
void launch_log(dim3 grid, dim3 block, size_t lds_bytes, const char* fmt, ...)
    __attribute__((format(printf, 4, 5)));

// Compute units of the calling thread's current device (cached per device; 256 when
// the query fails).
int device_compute_units();

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

// Whether the matrix-core small-M GEMV takes M rows at this K and code width (M <= 8).
bool qmv_mfma_takes(int64_t K, int bits, int64_t M);

// Matrix-core GEMM for M >= 8.
hipError_t launch_qmm_mfma(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
                           const uint16_t* biases, void* y, int64_t M, int64_t N, int64_t K,
                           int bits, int group, bool out_f32, hipStream_t stream);

// Expert-gathered GEMM: prepare (validation + per-expert offsets into workspace),
// then the grouped matrix-core kernel. The status word also goes to `status` if not null.
size_t gather_workspace_bytes(int64_t E);
hipError_t launch_gather_qmm(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
                             const uint16_t* biases, const int32_t* expert_idx, void* y,
                             int64_t B, int64_t N, int64_t K, int64_t E, int bits, int group,
                             bool out_f32, void* workspace, hipStream_t stream,
                             uint32_t* status = nullptr);

// The same with the library's per-GPU static workspace (no allocation, no workspace
// argument); E at most gather_noalloc_max_experts().
int64_t gather_noalloc_max_experts();
hipError_t launch_gather_qmm_noalloc(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
                                     const uint16_t* biases, const int32_t* expert_idx, void* y,
                                     int64_t B, int64_t N, int64_t K, int64_t E, int bits, int group,
                                     bool out_f32, uint32_t* status, hipStream_t stream);

// Indexed GatherQMM (rows in any order, optional token index): a counting sort of the
// rows by expert into the workspace, then the grouped GEMM over the sorted rows.
size_t gather_indexed_workspace_bytes(int64_t B, int64_t E);
int64_t gather_indexed_max_experts();
hipError_t launch_gather_qmm_indexed(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
                                     const uint16_t* biases, const int32_t* token_idx,
                                     const int32_t* expert_idx, void* y, int64_t B, int64_t N,
                                     int64_t K, int64_t E, int64_t T, int bits, int group,
                                     bool out_f32, void* workspace, hipStream_t stream);

// Counting sort of B output rows by expert into the indexed-gather workspace layout
// (word 0 status, offsets [E+1], permutation [B]); rows with an out-of-range token or
// expert id are written as zeros in y (ysz bytes per element).
hipError_t launch_gather_sort(const int32_t* token_idx, const int32_t* expert_idx, int64_t B,
                              int64_t E, int64_t T, int64_t N, int ysz, void* y, void* workspace,
                              hipStream_t stream);

// Dense grouped product (gather_mm): the counting sort above, then the grouped
// matrix-core kernel over bf16 (dtype 0) or binary16 (dtype 1) operands, W stored
// [E, N, K] (layout 0) or [E, K, N] (layout 1); otype 0 bf16, 1 f32, 2 binary16.
hipError_t launch_gather_mm(const uint16_t* x, const uint16_t* w, const int32_t* token_idx,
                            const int32_t* expert_idx, void* y, int64_t B, int64_t N, int64_t K,
                            int64_t E, int64_t T, int dtype, int layout, int otype,
                            void* workspace, hipStream_t stream);

}  // namespace bitmm
