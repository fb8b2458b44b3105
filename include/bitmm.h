/*
 * bitmm: affine group-wise quantized matrix multiply on AMD Instinct MI355X (gfx950).
 *
 * The operation. The epic "NVIDIA Volta (sm_70) inference acceleration program"
 * (mlxcel #1536) profiles an inference engine whose GPU time is dominated by two
 * quantized-weight kernels: the prefill GEMM (its kernel table's first row) and
 * the decode GEMV (second row). Its Baseline section describes the weights as
 * affine quantized, 4-bit codes in groups of 64, with every other tensor in bf16;
 * issue #1538 ("Volta (sm_70) baseline record and build coverage", comments of
 * 2026-08-31) adds 8-bit codes; 2-bit codes, the narrowest width of the same format,
 * are packed by the same rule. PR #1562 ("tag the pre-Ampere grouped GEMM arm
 * Sm70, not Sm75", section "The branch is live") adds the third form: the
 * quantized GatherQMM that a MoE prefill runs over rows sorted by expert. All
 * three compute
 *
 *     y[r][n] = sum_k x[r][k] * w[e_r][n][k],
 *     w[e][n][k] = s[e][n][k/gs] * q[e][n][k] + b[e][n][k/gs],   gs = group_size,
 *
 * with e_r = 0 for the dense forms and e_r = expert_idx[r] for the gathered one. The
 * same PR's non-quantized MoE path, gather_mm, is bitmm_gather_mm at the end of this
 * file: the grouped product over plain bf16 or binary16 weights.
 *
 * Storage (all row-major, contiguous, little-endian):
 *   x        bf16 [M, K]                 (activations; bf16 passed as uint16 bits)
 *   w        uint32 [E, N, K*bits/32]    (codes along K, LSB first: code j of a word
 *                                         sits in bits [bits*j, bits*(j+1)) and word i
 *                                         of a row holds k = i*(32/bits) + j)
 *   scales   bf16 [E, N, K/group_size]   (one scale per row n and group along K)
 *   biases   bf16 [E, N, K/group_size]
 *   y        bf16 or f32 [M, N]          (bf16 rounded to nearest even from f32)
 * Dense calls have E = 1 and no leading E dimension.
 *
 * Precision. Accumulation is always f32 (the pages' decode fix, PR #1539 in the
 * epic's sub-issue list, is to stop accumulating the 4-bit GEMV in bf16).
 *   - bitmm_qmv, and bitmm_qmm on the GEMV kernels (M < 8, and M = 8 where the
 *     matrix-core GEMV takes it): every product x*w is formed exactly (the code enters
 *     as an exact bf16 integer and the group scale is applied in f32).
 *   - bitmm_qmm on the matrix-core GEMM and bitmm_gather_qmm: w = fma(s, q, b) in f32 is rounded
 *     to bf16 and multiplied on the matrix cores (a dense bf16 GEMM after
 *     dequantization, as the grouped path on the pages is), f32 accumulate.
 *
 * Conventions.
 *   - Pointers are DEVICE pointers owned by the caller; nothing is retained after
 *     the call returns and the library allocates no memory (the one exception,
 *     bitmm_gather_qmm_noalloc, uses a fixed 64 KiB array that the library holds per
 *     GPU from load time on).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and the
 *     call returns without synchronising. Calls are re-entrant and may run
 *     concurrently on different streams. Results are bitwise deterministic.
 *   - Arguments are validated on the host before any HIP call; a validation error
 *     enqueues nothing. M = 0, N = 0 or B = 0 is a valid empty problem (BITMM_OK,
 *     nothing enqueued, pointers unused).
 *   - No C++ exception crosses this interface.
 */
#ifndef BITMM_H
#define BITMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BITMM_ABI_VERSION 2

typedef enum {
  BITMM_OK = 0,
  BITMM_ERR_NULL = 1,        /* a required pointer is NULL                                  */
  BITMM_ERR_SHAPE = 2,       /* M, N, B < 0; K < 1; E < 1; K not a multiple of 64 and of
                                group_size                                                  */
  BITMM_ERR_UNSUPPORTED = 3, /* bits not in {2, 4, 8}; group_size not in {32, 64, 128}, or 32
                                with 2-bit codes; unknown
                                output type, operand type or layout; a size limit stated
                                at the entry point                                          */
  BITMM_ERR_ALIGN = 4,       /* x, w or workspace not 16-byte aligned; scales or biases not
                                2-byte aligned; y not aligned to its element size;
                                expert_idx not 4-byte aligned                               */
  BITMM_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than bitmm_gather_qmm_workspace_bytes */
  BITMM_ERR_DEVICE = 6,      /* no HIP device, or the current device is not gfx950          */
  BITMM_ERR_LAUNCH = 7       /* a kernel launch reported an error                           */
} bitmm_status;

/* Output element type. BITMM_OUT_F16 (IEEE binary16, rounded to nearest even) is
   accepted by bitmm_gather_mm only. */
typedef enum { BITMM_OUT_BF16 = 0, BITMM_OUT_F32 = 1, BITMM_OUT_F16 = 2 } bitmm_out;

/* Operand element type of bitmm_gather_mm (x and w alike). */
typedef enum { BITMM_DTYPE_BF16 = 0, BITMM_DTYPE_F16 = 1 } bitmm_dtype;

/* Storage of each expert's weight matrix for bitmm_gather_mm: [N, K] (one row per output
   column, K contiguous; the MoE layer's own layout) or [K, N] (N contiguous). */
typedef enum { BITMM_LAYOUT_NK = 0, BITMM_LAYOUT_KN = 1 } bitmm_layout;

/* Version of this interface (BITMM_ABI_VERSION), so a caller can check what it loaded
   before the first call. Plumbing, not an operation of the pages; its role matches the
   capability probe of issue #1537 that epic #1536 lists under "Phase 0" (the runtime
   asks what it is running against before choosing a path). */
int bitmm_abi_version(void);

/* Static, human-readable name of a status code ("unknown status" otherwise). Plumbing,
   not an operation of the pages: every failure comes back as a named status instead of
   an opaque launch failure, as issue #1538, comment "Baseline recorded: PR #1556"
   ("Build coverage decision") credits #1537 with doing for an architecture mismatch. */
const char* bitmm_status_string(bitmm_status s);

/*
 * Kernel-choice record: the kernels the calling thread's most recent bitmm_qmv, bitmm_qmm,
 * bitmm_gather_* call enqueued, one line each, "<kernel><template arguments> grid=XxY
 * block=T lds=B" (LDS bytes the kernel declares), in launch order; empty when that call
 * enqueued nothing (an error, or an empty problem). Copies at most len - 1 bytes and a
 * terminating NUL into buf (nothing if buf is NULL or len is 0) and returns the record's
 * full length. Host-only: no HIP call, no synchronisation. It names what the library
 * chose by shape, code width, group size and alignment (the pages' engine logs its
 * architecture decision for the same reason: epic #1536, "GB10 (sm_121) continuation",
 * the MLXCEL_TRACE_ARCH criterion of #1537).
 */
size_t bitmm_last_launches(char* buf, size_t len);

/*
 * Decode GEMV: y[M, N] = x[M, K] * dequant(w)^T, streaming W once per call for all M
 * rows (rows are taken eight at a time). Meant for M = 1 (the decode step the epic's
 * kernel table lists second); any M >= 0 is accepted.
 *   x: bf16 [M, K]; w: uint32 [N, K*bits/32]; scales, biases: bf16 [N, K/group_size];
 *   y: [M, N] of type `out`. bits in {2, 4, 8}; group_size in {32, 64, 128} (64 or 128
 *   at 2 bits, where one 16-byte chunk holds 64 codes; the epic's
 *   checkpoint is group 64; its diagnosis item 4 quotes a tile rule keyed on
 *   group_size <= 64, so other group sizes exist in the format); K a multiple of 64 and
 *   of group_size.
 * Limit (else BITMM_ERR_UNSUPPORTED): K <= 3355443 (byte offsets within a tile of up to 320
 * activation rows are 32-bit: 320 * K * 2 < 2^31). Same for bitmm_qmm.
 */
bitmm_status bitmm_qmv(const void* x, const uint32_t* w, const void* scales, const void* biases,
                       void* y, int64_t M, int64_t N, int64_t K, int bits, int group_size,
                       bitmm_out out, void* stream);

/*
 * Prefill GEMM: same operation and arguments as bitmm_qmv, for any M. Following the
 * engine's routing rule quoted in issue #1538 (the first 2026-08-31 comment: M*B >= 8
 * selects the GEMM), M < 8 runs the GEMV kernel (the small-M path) and M > 8 the
 * matrix-core GEMM; M = 8 stays on the GEMV where its matrix-core form takes the shape
 * (K <= 16384 at 4 bits, 8192 at 8, 32768 at 2), which is faster there. The choice of
 * kernel never changes what is computed.
 */
bitmm_status bitmm_qmm(const void* x, const uint32_t* w, const void* scales, const void* biases,
                       void* y, int64_t M, int64_t N, int64_t K, int bits, int group_size,
                       bitmm_out out, void* stream);

/*
 * Bytes of device workspace bitmm_gather_qmm needs for B rows, N columns and E experts
 * (a multiple of 256; 0 if an argument is negative or E < 1): the status word and the
 * per-expert row offsets, the data that the setup step of the grouped path produces
 * ahead of the grouped GEMM (PR #1562, "The branch is live": prepare_grouped_mm_data,
 * one per grouped-GEMM launch).
 */
size_t bitmm_gather_qmm_workspace_bytes(int64_t B, int64_t N, int64_t E);

/*
 * Expert-gathered GEMM (MoE prefill over rows sorted by expert; PR #1562):
 *   y[r, :] = x[r, :] * dequant(w[expert_idx[r]])^T for r in [0, B)
 *   x: bf16 [B, K]; w: uint32 [E, N, K*bits/32]; scales, biases: bf16 [E, N, K/group_size];
 *   expert_idx: int32 [B]; y: [B, N] of type `out`.
 * PRECONDITION: expert_idx is non-decreasing with every value in [0, E). This is checked
 * on the device: word 0 (uint32) of `workspace` receives 0 if it holds, otherwise 1 + the
 * first offending row, and then every row of y is written as zeros. Words 1..E+1 receive
 * the row offset of each expert (int32; expert e owns rows [off[e], off[e+1])). The caller
 * may read them back once the stream has reached this call; the library never waits.
 * `workspace` is caller-owned device memory of at least
 * bitmm_gather_qmm_workspace_bytes(B, N, E) bytes, 16-byte aligned; it needs no
 * initialisation. Two calls sharing one workspace must be ordered on one stream.
 */
bitmm_status bitmm_gather_qmm(const void* x, const uint32_t* w, const void* scales,
                              const void* biases, const int32_t* expert_idx, void* y, int64_t B,
                              int64_t N, int64_t K, int64_t E, int bits, int group_size,
                              bitmm_out out, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * bitmm_gather_qmm without a workspace argument and without any allocation, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. Same operation, arguments, precondition check and
 * results as bitmm_gather_qmm; the status word and the expert offsets go to a workspace
 * of 64 KiB that the library keeps in device memory, one per GPU, for the life of the
 * process (it holds whatever the last call left there; every word a call reads was
 * written earlier by the same call).
 *   status: optional device pointer (uint32, 4-byte aligned; NULL = not reported) that
 *           receives the status word: 0 if the precondition holds, otherwise 1 + the
 *           first offending row (y is then all zeros).
 * Limit: E <= 16382 (else BITMM_ERR_UNSUPPORTED). Every call on one GPU uses that GPU's
 * workspace, so calls that may overlap on one GPU (different streams without ordering)
 * race; order them on one stream, or use bitmm_gather_qmm with workspaces of their own.
 */
bitmm_status bitmm_gather_qmm_noalloc(const void* x, const uint32_t* w, const void* scales,
                                      const void* biases, const int32_t* expert_idx, void* y,
                                      int64_t B, int64_t N, int64_t K, int64_t E, int bits,
                                      int group_size, bitmm_out out, uint32_t* status,
                                      void* stream);

/*
 * Bytes of device workspace bitmm_gather_qmm_indexed needs for B rows, N columns and E
 * experts (a multiple of 256; 0 if an argument is negative or E < 1).
 */
size_t bitmm_gather_qmm_indexed_workspace_bytes(int64_t B, int64_t N, int64_t E);

/*
 * Indexed expert-gathered GEMM: the general GatherQMM of PR #1562 (its MoE layer
 * passes the activation rows through an index rather than replicating them per
 * expert), with rows in any order:
 *   y[r, :] = x[t_r, :] * dequant(w[expert_idx[r]])^T for r in [0, B),
 *   t_r = token_idx[r], or r when token_idx is NULL.
 *   x: bf16 [T, K]; w: uint32 [E, N, K*bits/32]; scales, biases: bf16 [E, N, K/group_size];
 *   token_idx (optional), expert_idx: int32 [B]; y: [B, N] of type `out`.
 * A first kernel groups the rows by expert (a counting sort into the workspace) and
 * writes zeros to every row whose token id is outside [0, T) or expert id outside
 * [0, E); the grouped GEMM then runs over the grouped rows, reading each activation row
 * through the index. Workspace word 0 (uint32) receives 0, or 1 + the first row with an
 * out-of-range id. `workspace`: caller-owned device memory of at least
 * bitmm_gather_qmm_indexed_workspace_bytes(B, N, E) bytes, 16-byte aligned, no
 * initialisation needed; two calls sharing it must be ordered on one stream.
 * Limits (else BITMM_ERR_UNSUPPORTED): E <= 8192; T * K * 2 < 2^31.
 * Precision as bitmm_gather_qmm.
 */
bitmm_status bitmm_gather_qmm_indexed(const void* x, const uint32_t* w, const void* scales,
                                      const void* biases, const int32_t* token_idx,
                                      const int32_t* expert_idx, void* y, int64_t B, int64_t N,
                                      int64_t K, int64_t E, int64_t T, int bits, int group_size,
                                      bitmm_out out, void* workspace, size_t workspace_bytes,
                                      void* stream);

/*
 * Gathered GEMV for MoE decode. Issue #1538's correction on MoE decode (its comment
 * "MoE decode does not route to qmm_naive") finds the decode-time experts running in
 * dedicated per-token kernels, apart from the prefill grouped GEMM; each of their
 * products is this one, the general GatherQMM of PR #1562 with one activation row per
 * output row:
 *   y[r, :] = x[t_r, :] * dequant(w[expert_idx[r]])^T for r in [0, B),
 *   t_r = token_idx[r], or r when token_idx is NULL.
 *   x: bf16 [T, K]; w: uint32 [E, N, K*bits/32]; scales, biases: bf16 [E, N, K/group_size];
 *   token_idx (optional), expert_idx: int32 [B], any order, repeats allowed;
 *   y: [B, N] of type `out`.
 * A row whose token id is outside [0, T) or whose expert id is outside [0, E) is written
 * as zeros. Each row streams its expert's weights once; no workspace, one launch (more
 * only past 65535 rows). Products are exact and accumulation f32, as in bitmm_qmv.
 */
bitmm_status bitmm_gather_qmv(const void* x, const uint32_t* w, const void* scales,
                              const void* biases, const int32_t* token_idx,
                              const int32_t* expert_idx, void* y, int64_t B, int64_t N, int64_t K,
                              int64_t E, int64_t T, int bits, int group_size, bitmm_out out,
                              void* stream);

/*
 * Bytes of device workspace bitmm_gather_mm needs for B rows, N columns and E experts
 * (a multiple of 256; 0 if an argument is negative or E < 1).
 */
size_t bitmm_gather_mm_workspace_bytes(int64_t B, int64_t N, int64_t E);

/*
 * Dense grouped product for non-quantized MoE layers (gather_mm). PR #1562 ("The branch
 * is live") notes that every non-quantized MoE checkpoint reaches the grouped GEMM
 * through SwitchLinear::Regular::forward, with no gate, and its tests check gather_mm
 * against an f64 dense per-expert product in both operand layouts and in f32, bf16 and
 * f16. The same scheduler as bitmm_gather_qmm_indexed, without dequantization:
 *   y[r, :] = x[t_r, :] * W[expert_idx[r]]^T for r in [0, B),
 *   t_r = token_idx[r], or r when token_idx is NULL.
 *   x: [T, K] and w: [E, N, K] (layout BITMM_LAYOUT_NK) or [E, K, N] (BITMM_LAYOUT_KN),
 *   both of type `dtype` (bf16 or binary16 bit patterns); token_idx (optional),
 *   expert_idx: int32 [B], any order, repeats allowed; y: [B, N] of type `out` (bf16,
 *   f32 or binary16, independent of `dtype`).
 * Products of the operands are exact in f32 and accumulation is f32 (matrix cores).
 * Rows with an out-of-range token or expert id are written as zeros and workspace word 0
 * (uint32) receives 1 + the first such row (0 if none). `workspace`: caller-owned device
 * memory of at least bitmm_gather_mm_workspace_bytes(B, N, E) bytes, 16-byte aligned, no
 * initialisation needed; two calls sharing it must be ordered on one stream.
 * Limits (else BITMM_ERR_UNSUPPORTED): K a multiple of 16; with BITMM_LAYOUT_KN, N a
 * multiple of 8; E <= 8192; T * K * 2 < 2^31 and N * K * 2 < 2^31 (one expert's weights).
 * f32 operands are not supported (BITMM_ERR_UNSUPPORTED for any other dtype).
 */
bitmm_status bitmm_gather_mm(const void* x, const void* w, const int32_t* token_idx,
                             const int32_t* expert_idx, void* y, int64_t B, int64_t N, int64_t K,
                             int64_t E, int64_t T, bitmm_dtype dtype, bitmm_layout layout,
                             bitmm_out out, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BITMM_H */
