/*
 * CPU oracle for the affine group-wise quantized matmul and the dense grouped
 * product (gather_mm): test infrastructure
 * only (tests, smoke check, benchmark CPU baseline). See oracle.c for the
 * definition it follows and the readings it takes.
 *
 * All tensors are host arrays, row-major. bf16 values are passed as their
 * uint16 bit patterns. Outputs are double. Functions returning int return the
 * number of threads used, or a negative value for invalid arguments.
 * nthreads <= 0 means every core in the process affinity mask.
 */
#ifndef BITMM_ORACLE_H
#define BITMM_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

double oracle_bf16_to_f64(uint16_t h);
uint16_t oracle_f64_to_bf16_rne(double v);
void oracle_f64_to_bf16_array(const double* v, uint16_t* out, int64_t n);
double oracle_f16_to_f64(uint16_t h); /* IEEE binary16 bit pattern, exact */
uint16_t oracle_f64_to_f16_rne(double v);
void oracle_f64_to_f16_array(const double* v, uint16_t* out, int64_t n);
void oracle_f16_to_f64_array(const uint16_t* h, double* out, int64_t n);
uint32_t oracle_code(const uint32_t* row_words, int64_t k, int bits);
double oracle_weight(const uint32_t* row_words, const uint16_t* row_scales,
                     const uint16_t* row_biases, int64_t k, int bits, int group);
int oracle_default_threads(void);

/* y[M*N] = x[M,K] . dequant(w[N, K*bits/32])^T */
int oracle_qmm(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
               const uint16_t* biases, int64_t M, int64_t N, int64_t K, int bits, int group,
               double* y, int nthreads);

/* y[i] = output (rows[i], cols[i]) of the same problem */
int oracle_qmm_points(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
                      const uint16_t* biases, int64_t M, int64_t N, int64_t K, int bits,
                      int group, const int64_t* rows, const int64_t* cols, int64_t count,
                      double* y, int nthreads);

/* y[B*N]: row r uses expert expert_idx[r] of w[E, N, K*bits/32] (zero row if out of range) */
int oracle_gather_qmm(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
                      const uint16_t* biases, const int32_t* expert_idx, int64_t B, int64_t N,
                      int64_t K, int64_t E, int bits, int group, double* y, int nthreads);

int oracle_gather_qmm_points(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
                             const uint16_t* biases, const int32_t* expert_idx, int64_t B,
                             int64_t N, int64_t K, int64_t E, int bits, int group,
                             const int64_t* rows, const int64_t* cols, int64_t count, double* y,
                             int nthreads);

/* y[B*N]: row r reads x row token_idx[r] of x[T, K] (row r when token_idx is NULL)
   and expert expert_idx[r] of w; any order; zero row if either id is out of range */
int oracle_gather_qmm_indexed(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
                              const uint16_t* biases, const int32_t* token_idx,
                              const int32_t* expert_idx, int64_t B, int64_t N, int64_t K,
                              int64_t E, int64_t T, int bits, int group, double* y, int nthreads);

int oracle_gather_qmm_indexed_points(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
                                     const uint16_t* biases, const int32_t* token_idx,
                                     const int32_t* expert_idx, int64_t B, int64_t N, int64_t K,
                                     int64_t E, int64_t T, int bits, int group, const int64_t* rows,
                                     const int64_t* cols, int64_t count, double* y, int nthreads);

/* Dense grouped product: y[B*N], row r reads x row token_idx[r] of x[T, K] (row r
   when token_idx is NULL) and the weights of expert expert_idx[r]; W is [E, N, K]
   (layout 0) or [E, K, N] (layout 1); x and W are bf16 (dtype 0) or binary16
   (dtype 1) bit patterns; zero row if either id is out of range */
int oracle_gather_mm(const uint16_t* x, const uint16_t* w, const int32_t* token_idx,
                     const int32_t* expert_idx, int64_t B, int64_t N, int64_t K, int64_t E,
                     int64_t T, int dtype, int layout, double* y, int nthreads);

int oracle_gather_mm_points(const uint16_t* x, const uint16_t* w, const int32_t* token_idx,
                            const int32_t* expert_idx, int64_t B, int64_t N, int64_t K, int64_t E,
                            int64_t T, int dtype, int layout, const int64_t* rows,
                            const int64_t* cols, int64_t count, double* y, int nthreads);

#ifdef __cplusplus
}
#endif

#endif
