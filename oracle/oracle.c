/*
 * CPU oracle for the affine group-wise quantized matmul and the dense grouped
 * product beside it (gather_mm). TEST INFRASTRUCTURE
 * ONLY: the tests, the smoke check and the benchmark's CPU-baseline leg use it.
 * The library never calls, links or loads it, and it shares no code with the
 * HIP kernels.
 *
 * What it computes. The epic "NVIDIA Volta (sm_70) inference acceleration
 * program" (#1536), Baseline section, describes the checkpoints as affine
 * quantized with 4-bit codes in groups of 64 and every other tensor in bf16;
 * its kernel table names the code type (CUTLASS 4-bit sub-byte integers), and
 * issue #1538 ("Volta (sm_70) baseline record and build coverage", comment of
 * 2026-08-31) sets those against 8-bit unsigned-char codes. 2-bit codes, the
 * narrowest width of the same affine format, are packed the same way (16 per
 * word). So:
 *
 *   for each output row r and column n
 *     y[r][n] = sum_k x[r][k] * (s[n][g] * q[n][k] + b[n][g]),  g = floor(k / group)
 *
 * with x, s, b bf16 values widened exactly, q the unsigned code stored in the
 * packed word, and every step in double precision. The grouped variant (PR
 * #1562, "tag the pre-Ampere grouped GEMM arm Sm70, not Sm75", section "The
 * branch is live": the quantized GatherQMM over rows sorted by expert) uses
 * the weight slab of expert e_r = expert_idx[r] for row r. Where the pages
 * leave a step open, the readings used are:
 *   - dequantization is w = s*q + b with unsigned codes and no separate zero
 *     point; s and b come from the group floor(k/group) of the same row n;
 *   - codes are packed LSB first: code j of a uint32 occupies bits
 *     [bits*j, bits*(j+1)), and word i of a row holds k = i*(32/bits) + j;
 *   - W is stored [N, K] (one row per output feature), so y = x * W^T;
 *   - accumulation is at least f32 (the pages' fix for the 4-bit GEMV is to
 *     stop accumulating in bf16); the oracle uses f64, the exact definition.
 * A row whose expert id lies outside [0, E) contributes a zero row.
 *
 * The indexed form is the general GatherQMM the pages name (PR #1562: the MoE
 * layer's quantized GatherQMM; epic #1536 and issue #1538: the decode-time expert
 * kernels that run the same product one token at a time): row r of the output
 * reads activation row token_idx[r] of x[T, K] (row r itself when no token index
 * is given) and the weights of expert expert_idx[r], in any order. A row whose
 * token or expert id is out of range is a zero row.
 *
 * The dense grouped product (gather_mm) is the same scheduler without the
 * dequantization step (PR #1562: non-quantized MoE checkpoints reach the grouped
 * GEMM through SwitchLinear::Regular::forward, and its new tests compare gather_mm
 * with an f64 dense per-expert product in both operand layouts, in f32, bf16 and
 * f16): row r of the output is
 *
 *   y[r][n] = sum_k x[t_r][k] * W[e_r][n][k]      (weights stored [E, N, K])
 *   y[r][n] = sum_k x[t_r][k] * W[e_r][k][n]      (weights stored [E, K, N])
 *
 * with x and W both bf16 or both IEEE binary16, widened exactly.
 *
 * Each output is summed sequentially in k order, and threads only split the
 * set of outputs, so results are bitwise identical for any thread count.
 *
 * Every function here is pinned by the CPU test-suite (brute force against an
 * independent numpy path, integer-exact cases, closed forms, a constant-per-
 * expert case and printed bf16 bit patterns); none is "parity unpinned".
 */
#define _GNU_SOURCE
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <string.h>
#include <time.h>
#include <unistd.h>

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
double oracle_bf16_to_f64(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Exponent field 0 holds zero and the subnormals f * 2^-24; field 31 holds the
 * infinities (f = 0) and NaNs. Widening to double is exact. */
double oracle_f16_to_f64(uint16_t h) {
  int sign = h >> 15;
  int field = (h >> 10) & 0x1F;
  int frac = h & 0x3FF;
  double v;
  if (field == 0)
    v = ldexp((double)frac, -24);
  else if (field == 31)
    v = frac ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + frac), field - 25);
  return sign ? -v : v;
}

/* Round a double to the nearest binary16, ties to even, in one step: the same
 * construction as the bf16 rounding below with a 10-bit fraction, exponent bias
 * 15 and subnormal step 2^-24. */
uint16_t oracle_f64_to_f16_rne(double v) {
  uint16_t sign = signbit(v) ? 0x8000u : 0u;
  double a = fabs(v);
  if (isnan(v)) return (uint16_t)(sign | 0x7E00u);
  if (isinf(v)) return (uint16_t)(sign | 0x7C00u);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
  if (e - 1 < -14) {
    /* subnormal: value = r * 2^-24, r in [0, 1024]; r == 1024 is the smallest
     * normal, whose encoding is also 1024. */
    double r = nearbyint(ldexp(a, 24));
    return (uint16_t)(sign | (uint16_t)r);
  }
  double r = nearbyint(ldexp(a, 11 - e)); /* in [1024, 2048] */
  if (r == 2048.0) {
    r = 1024.0;
    e += 1;
  }
  int biased = e - 1 + 15;
  if (biased >= 31) return (uint16_t)(sign | 0x7C00u);
  return (uint16_t)(sign | (uint16_t)(biased << 10) | (uint16_t)((int)r - 1024));
}

/* Round a double to the nearest bf16, ties to even, in one step (no detour
 * through float). Overflow goes to infinity, NaN to a quiet NaN, values below
 * the normal range to bf16 subnormals. */
uint16_t oracle_f64_to_bf16_rne(double v) {
  uint16_t sign = signbit(v) ? 0x8000u : 0u;
  double a = fabs(v);
  if (isnan(v)) return (uint16_t)(sign | 0x7FC0u);
  if (isinf(v)) return (uint16_t)(sign | 0x7F80u);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
  if (e - 1 < -126) {
    /* subnormal bf16: value = r * 2^-133, r in [0, 128]; r == 128 is the
     * smallest normal, whose encoding is also 128. */
    double r = nearbyint(ldexp(a, 133));
    return (uint16_t)(sign | (uint16_t)r);
  }
  double r = nearbyint(ldexp(a, 8 - e)); /* in [128, 256] */
  if (r == 256.0) {
    r = 128.0;
    e += 1;
  }
  int biased = e - 1 + 127;
  if (biased >= 255) return (uint16_t)(sign | 0x7F80u);
  return (uint16_t)(sign | (uint16_t)(biased << 7) | (uint16_t)((int)r - 128));
}

/* The code for element k of a packed row (LSB-first layout). */
uint32_t oracle_code(const uint32_t* row_words, int64_t k, int bits) {
  int64_t per_word = 32 / bits;
  uint32_t word = row_words[k / per_word];
  int pos = (int)(k % per_word);
  uint32_t mask = (1u << bits) - 1u;
  return (word >> (bits * pos)) & mask;
}

/* The dequantized weight w[n][k] = s[n][g] * q[n][k] + b[n][g]. */
double oracle_weight(const uint32_t* row_words, const uint16_t* row_scales,
                     const uint16_t* row_biases, int64_t k, int bits, int group) {
  int64_t g = k / group;
  double q = (double)oracle_code(row_words, k, bits);
  return oracle_bf16_to_f64(row_scales[g]) * q + oracle_bf16_to_f64(row_biases[g]);
}

/* One output: sum over k of x[k] * w[n][k], in k order, in double. */
static double dot_row(const uint16_t* x_row, const uint32_t* w_row, const uint16_t* s_row,
                      const uint16_t* b_row, int64_t K, int bits, int group) {
  double acc = 0.0;
  for (int64_t k = 0; k < K; ++k)
    acc += oracle_bf16_to_f64(x_row[k]) * oracle_weight(w_row, s_row, b_row, k, bits, group);
  return acc;
}

/* ------------------------------------------------------------------------ */
/* A generic problem description: output (r, n) reads x row r and the weight */
/* row n of expert sel(r); sel = 0 for the dense case.                        */

typedef struct {
  const uint16_t* x;
  const uint32_t* w;
  const uint16_t* s;
  const uint16_t* b;
  const int32_t* expert_idx; /* NULL for the dense case */
  const int32_t* token_idx;  /* NULL: output row r reads activation row r */
  int64_t N, K, E, T;
  int bits, group;
  /* outputs: either all rows x cols, or a list of points */
  int64_t rows;
  const int64_t* pt_r;
  const int64_t* pt_n;
  int64_t count; /* number of outputs */
  double* y;
} problem_t;

static double eval_point(const problem_t* p, int64_t r, int64_t n) {
  int64_t words = p->K * p->bits / 32;
  int64_t groups = p->K / p->group;
  int64_t e = 0;
  if (p->expert_idx) {
    e = p->expert_idx[r];
    if (e < 0 || e >= p->E) return 0.0;
  }
  int64_t t = r;
  if (p->token_idx) {
    t = p->token_idx[r];
    if (t < 0 || t >= p->T) return 0.0;
  }
  const uint32_t* w_row = p->w + (e * p->N + n) * words;
  const uint16_t* s_row = p->s + (e * p->N + n) * groups;
  const uint16_t* b_row = p->b + (e * p->N + n) * groups;
  return dot_row(p->x + t * p->K, w_row, s_row, b_row, p->K, p->bits, p->group);
}

typedef struct {
  const problem_t* p;
  int64_t begin, end;
} slice_t;

static void* run_slice(void* arg) {
  const slice_t* sl = (const slice_t*)arg;
  const problem_t* p = sl->p;
  for (int64_t i = sl->begin; i < sl->end; ++i) {
    int64_t r, n;
    if (p->pt_r) {
      r = p->pt_r[i];
      n = p->pt_n[i];
    } else {
      r = i / p->N;
      n = i % p->N;
    }
    p->y[i] = eval_point(p, r, n);
  }
  return NULL;
}

int oracle_default_threads(void) {
  cpu_set_t set;
  if (sched_getaffinity(0, sizeof set, &set) == 0) {
    int c = CPU_COUNT(&set);
    if (c > 0) return c;
  }
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  return n > 0 ? (int)n : 1;
}

#define ORACLE_MAX_THREADS 256

static int run(const problem_t* p, int nthreads) {
  if (nthreads <= 0) nthreads = oracle_default_threads();
  if (nthreads > ORACLE_MAX_THREADS) nthreads = ORACLE_MAX_THREADS;
  if ((int64_t)nthreads > p->count) nthreads = p->count > 0 ? (int)p->count : 1;
  pthread_t tid[ORACLE_MAX_THREADS];
  slice_t sl[ORACLE_MAX_THREADS];
  int64_t chunk = (p->count + nthreads - 1) / nthreads;
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    sl[t].p = p;
    sl[t].begin = (int64_t)t * chunk;
    sl[t].end = sl[t].begin + chunk < p->count ? sl[t].begin + chunk : p->count;
    if (sl[t].begin >= sl[t].end) break;
    if (t == 0) continue; /* slice 0 runs on the calling thread */
    if (pthread_create(&tid[t], NULL, run_slice, &sl[t]) != 0) {
      run_slice(&sl[t]); /* could not spawn: do it here */
      tid[t] = 0;
    }
    started = t + 1;
  }
  if (p->count > 0) run_slice(&sl[0]);
  for (int t = 1; t < started; ++t)
    if (tid[t]) pthread_join(tid[t], NULL);
  return nthreads;
}

static int check_args(int64_t N, int64_t K, int bits, int group) {
  if (bits != 2 && bits != 4 && bits != 8) return -1;
  if (group <= 0 || K <= 0 || N < 0 || K % group != 0 || (K * bits) % 32 != 0) return -1;
  return 0;
}

int oracle_qmm(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
               const uint16_t* biases, int64_t M, int64_t N, int64_t K, int bits, int group,
               double* y, int nthreads) {
  if (M < 0 || check_args(N, K, bits, group)) return -1;
  problem_t p = {x, w, scales, biases, NULL, NULL, N, K, 1, M, bits, group, M, NULL, NULL, M * N, y};
  return run(&p, nthreads);
}

int oracle_qmm_points(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
                      const uint16_t* biases, int64_t M, int64_t N, int64_t K, int bits,
                      int group, const int64_t* rows, const int64_t* cols, int64_t count,
                      double* y, int nthreads) {
  if (M < 0 || count < 0 || check_args(N, K, bits, group)) return -1;
  for (int64_t i = 0; i < count; ++i)
    if (rows[i] < 0 || rows[i] >= M || cols[i] < 0 || cols[i] >= N) return -2;
  problem_t p = {x, w, scales, biases, NULL, NULL, N, K, 1, M, bits, group, M, rows, cols, count, y};
  return run(&p, nthreads);
}

int oracle_gather_qmm(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
                      const uint16_t* biases, const int32_t* expert_idx, int64_t B, int64_t N,
                      int64_t K, int64_t E, int bits, int group, double* y, int nthreads) {
  if (B < 0 || E < 1 || check_args(N, K, bits, group)) return -1;
  problem_t p = {x, w, scales, biases, expert_idx, NULL, N, K, E, B, bits, group, B, NULL, NULL, B * N, y};
  return run(&p, nthreads);
}

int oracle_gather_qmm_points(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
                             const uint16_t* biases, const int32_t* expert_idx, int64_t B,
                             int64_t N, int64_t K, int64_t E, int bits, int group,
                             const int64_t* rows, const int64_t* cols, int64_t count, double* y,
                             int nthreads) {
  if (B < 0 || E < 1 || count < 0 || check_args(N, K, bits, group)) return -1;
  for (int64_t i = 0; i < count; ++i)
    if (rows[i] < 0 || rows[i] >= B || cols[i] < 0 || cols[i] >= N) return -2;
  problem_t p = {x, w, scales, biases, expert_idx, NULL, N, K, E, B, bits, group, B, rows, cols, count, y};
  return run(&p, nthreads);
}

int oracle_gather_qmm_indexed(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
                              const uint16_t* biases, const int32_t* token_idx,
                              const int32_t* expert_idx, int64_t B, int64_t N, int64_t K,
                              int64_t E, int64_t T, int bits, int group, double* y, int nthreads) {
  if (B < 0 || E < 1 || T < 0 || check_args(N, K, bits, group)) return -1;
  problem_t p = {x, w, scales, biases, expert_idx, token_idx, N, K, E, T, bits, group, B, NULL, NULL, B * N, y};
  return run(&p, nthreads);
}

int oracle_gather_qmm_indexed_points(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
                                     const uint16_t* biases, const int32_t* token_idx,
                                     const int32_t* expert_idx, int64_t B, int64_t N, int64_t K,
                                     int64_t E, int64_t T, int bits, int group, const int64_t* rows,
                                     const int64_t* cols, int64_t count, double* y, int nthreads) {
  if (B < 0 || E < 1 || T < 0 || count < 0 || check_args(N, K, bits, group)) return -1;
  for (int64_t i = 0; i < count; ++i)
    if (rows[i] < 0 || rows[i] >= B || cols[i] < 0 || cols[i] >= N) return -2;
  problem_t p = {x, w, scales, biases, expert_idx, token_idx, N, K, E, T, bits, group, B, rows, cols, count, y};
  return run(&p, nthreads);
}

void oracle_f64_to_bf16_array(const double* v, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_bf16_rne(v[i]);
}

void oracle_f64_to_f16_array(const double* v, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_f16_rne(v[i]);
}

void oracle_f16_to_f64_array(const uint16_t* h, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f64(h[i]);
}

/* ------------------------------------------------------------------------ */
/* Dense grouped product (gather_mm).                                        */

typedef struct {
  const uint16_t* x;
  const uint16_t* w;
  const int32_t* token_idx; /* NULL: output row r reads activation row r */
  const int32_t* expert_idx;
  int64_t N, K, E, T;
  int dtype;  /* 0: bf16, 1: binary16 */
  int layout; /* 0: W[e] is [N, K]; 1: W[e] is [K, N] */
  const int64_t* pt_r;
  const int64_t* pt_n;
  int64_t count;
  double* y;
} dense_problem_t;

static double operand(uint16_t h, int dtype) {
  return dtype == 0 ? oracle_bf16_to_f64(h) : oracle_f16_to_f64(h);
}

static double dense_point(const dense_problem_t* p, int64_t r, int64_t n) {
  int64_t e = p->expert_idx[r];
  if (e < 0 || p->E <= e) return 0.0;
  int64_t t = r;
  if (p->token_idx) {
    t = p->token_idx[r];
    if (t < 0 || p->T <= t) return 0.0;
  }
  const uint16_t* x_row = p->x + p->K * t;
  const uint16_t* we = p->w + e * p->N * p->K;
  double acc = 0.0;
  for (int64_t k = 0; k < p->K; ++k) {
    uint16_t wv = p->layout == 0 ? we[n * p->K + k] : we[k * p->N + n];
    acc += operand(x_row[k], p->dtype) * operand(wv, p->dtype);
  }
  return acc;
}

typedef struct {
  const dense_problem_t* p;
  int64_t begin, end;
} dense_slice_t;

static void* run_dense_slice(void* arg) {
  const dense_slice_t* sl = (const dense_slice_t*)arg;
  const dense_problem_t* p = sl->p;
  for (int64_t i = sl->begin; i < sl->end; ++i) {
    int64_t r = p->pt_r ? p->pt_r[i] : i / p->N;
    int64_t n = p->pt_r ? p->pt_n[i] : i % p->N;
    p->y[i] = dense_point(p, r, n);
  }
  return NULL;
}

static int run_dense(const dense_problem_t* p, int nthreads) {
  if (nthreads <= 0) nthreads = oracle_default_threads();
  if (nthreads > ORACLE_MAX_THREADS) nthreads = ORACLE_MAX_THREADS;
  if ((int64_t)nthreads > p->count) nthreads = p->count > 0 ? (int)p->count : 1;
  pthread_t tid[ORACLE_MAX_THREADS];
  dense_slice_t sl[ORACLE_MAX_THREADS];
  int64_t chunk = (p->count + nthreads - 1) / nthreads;
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    sl[t].p = p;
    sl[t].begin = (int64_t)t * chunk;
    sl[t].end = sl[t].begin + chunk < p->count ? sl[t].begin + chunk : p->count;
    if (sl[t].begin >= sl[t].end) break;
    if (t == 0) continue;
    if (pthread_create(&tid[t], NULL, run_dense_slice, &sl[t]) != 0) {
      run_dense_slice(&sl[t]);
      tid[t] = 0;
    }
    started = t + 1;
  }
  if (p->count > 0) run_dense_slice(&sl[0]);
  for (int t = 1; t < started; ++t)
    if (tid[t]) pthread_join(tid[t], NULL);
  return nthreads;
}

int oracle_gather_mm(const uint16_t* x, const uint16_t* w, const int32_t* token_idx,
                     const int32_t* expert_idx, int64_t B, int64_t N, int64_t K, int64_t E,
                     int64_t T, int dtype, int layout, double* y, int nthreads) {
  if (B < 0 || N < 0 || K < 1 || E < 1 || T < 0 || (dtype != 0 && dtype != 1) ||
      (layout != 0 && layout != 1))
    return -1;
  dense_problem_t p = {x, w, token_idx, expert_idx, N, K, E, T, dtype, layout, NULL, NULL, B * N, y};
  return run_dense(&p, nthreads);
}

int oracle_gather_mm_points(const uint16_t* x, const uint16_t* w, const int32_t* token_idx,
                            const int32_t* expert_idx, int64_t B, int64_t N, int64_t K, int64_t E,
                            int64_t T, int dtype, int layout, const int64_t* rows,
                            const int64_t* cols, int64_t count, double* y, int nthreads) {
  if (B < 0 || N < 0 || K < 1 || E < 1 || T < 0 || count < 0 || (dtype != 0 && dtype != 1) ||
      (layout != 0 && layout != 1))
    return -1;
  for (int64_t i = 0; i < count; ++i)
    if (rows[i] < 0 || rows[i] >= B || cols[i] < 0 || cols[i] >= N) return -2;
  dense_problem_t p = {x, w, token_idx, expert_idx, N, K, E, T, dtype, layout, rows, cols, count, y};
  return run_dense(&p, nthreads);
}
