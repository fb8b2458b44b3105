// Expert-gathered GEMM for MoE prefill: y[r, :] = x[r, :] * dequant(w[e_r])^T with the
// rows sorted by expert (PR #1562, section "The branch is live": the sorted-MoE fast
// path hands a quantized GatherQMM to a grouped GEMM once the batch reaches
// min_rows * num_experts rows, and that GEMM is preceded by one setup kernel,
// prepare_grouped_mm_data, per launch).
//
// Two kernels on the caller's stream:
//   1. prepare (one workgroup): checks the precondition (ids non-decreasing and in
//      [0, E)), writes the status word and the per-expert row offsets into the
//      caller's workspace.
//   2. grouped GEMM: one workgroup per (expert, column block). It reads its expert's
//      row range from the workspace and runs the shared matrix-core tile over those
//      rows, so each expert's codes are streamed once per column block however many
//      rows the expert has. Experts without rows exit at once.
#include <atomic>
#include <mutex>

#include "kernels.hpp"
#include "mfma_tile4.hpp"

namespace bitmm {
namespace {

constexpr int kPrepThreads = 1024;
constexpr int kPrepRun = 8;  // rows per thread whose ids are loaded together

// ws[0]: 0 if the ids are valid, else 1 + first offending row.
// ws[1 + e], e in [0, E]: first row whose id is >= e (row offsets of the experts).
// One pass over the ids, every thread on rows t, t + 1024, ...: where the id steps up
// from a (the previous row's id, -1 before row 0) to c, the offsets of the experts
// a+1 .. c are that row; past the last row, the offsets of the experts after its id
// are B. With valid ids each offset is written exactly once; with invalid ones the
// offsets are not meaningful and the grouped GEMM does not read them. The status word
// is also written to `status` when that is not null.
__global__ __launch_bounds__(kPrepThreads) void gather_prepare_kernel(const int32_t* __restrict__ idx,
                                                                      int B, int E,
                                                                      uint32_t* __restrict__ ws,
                                                                      uint32_t* __restrict__ status) {
  __shared__ int first_bad;
  if (threadIdx.x == 0) first_bad = B;
  __syncthreads();
  int32_t* off = reinterpret_cast<int32_t*>(ws + 1);
  int mine = B;
  // kPrepRun rows per thread and pass, all their ids loaded before any is used: one
  // memory latency per pass instead of one per row.
  for (int base = 0; base < B; base += kPrepThreads * kPrepRun) {
    int cv[kPrepRun], av[kPrepRun];
    // Unconditional loads (rows past the end re-read the last one and are not used): a
    // load under a condition would be waited for where the paths join.
#pragma unroll
    for (int k = 0; k < kPrepRun; ++k) {
      const int r = min(base + (int)threadIdx.x + k * kPrepThreads, B - 1);
      cv[k] = idx[r];
      av[k] = idx[max(r - 1, 0)];
    }
#pragma unroll
    for (int k = 0; k < kPrepRun; ++k) {
      const int r = base + (int)threadIdx.x + k * kPrepThreads;
      if (r >= B) break;
      const int c = cv[k], a = r > 0 ? av[k] : -1;
      if (c < 0 || c >= E || a > c) {
        mine = min(mine, r);
        continue;
      }
      for (int e = max(a, -1) + 1; e <= c; ++e) off[e] = r;  // a may be an invalid id
    }
  }
  if (B > 0 && threadIdx.x == 0) {
    const int last = idx[B - 1];
    for (int e = max(last, -1) + 1; e <= E; ++e) off[e] = B;
  }
  if (B == 0)
    for (int e = threadIdx.x; e <= E; e += kPrepThreads) off[e] = 0;
  if (mine < B) atomicMin(&first_bad, mine);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t v = first_bad < B ? (uint32_t)first_bad + 1u : 0u;
    ws[0] = v;
    if (status) *status = v;
  }
}

// Indexed form: rows in any order, an optional token index. One workgroup builds a
// permutation that groups the rows by expert (a counting sort; the order of rows within
// an expert does not matter, since every output row is computed on its own) and zeros
// the output rows whose token or expert id is out of range. Workspace words:
//   [0]                 0, or 1 + the first row with an out-of-range id;
//   [1 .. E+1]          offsets: expert e owns perm[off[e] .. off[e+1]);
//   [E+2 .. E+2+B)      perm: output rows grouped by expert (invalid rows at the end).
constexpr int kMaxIndexedExperts = 8192;  // per-expert counters live in LDS

// Exclusive prefix sum of v[0 .. n) in LDS, in place, by all kPrepThreads threads:
// each thread sums a run of entries, the run totals are scanned within each wave with
// lane shifts and across the waves by one wave, then each thread rewrites its run.
__device__ void block_exclusive_scan(int* v, int n, int* part) {
  constexpr int kWaves = kPrepThreads / 64;
  const int per = (n + kPrepThreads - 1) / kPrepThreads;
  const int b0 = min(n, (int)threadIdx.x * per), b1 = min(n, b0 + per);
  int t = 0;
  for (int i = b0; i < b1; ++i) t += v[i];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = t;
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(inc, d, 64);
    if (lane >= d) inc += u;
  }
  if (lane == 63) part[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kWaves ? part[lane] : 0;
    for (int d = 1; d < kWaves; d <<= 1) {
      const int u = __shfl_up(w, d, 64);
      if (lane >= d) w += u;
    }
    if (lane < kWaves) part[kWaves + lane] = w;  // inclusive sums of the wave totals
  }
  __syncthreads();
  int acc = (wave > 0 ? part[kWaves + wave - 1] : 0) + inc - t;
  for (int i = b0; i < b1; ++i) {
    const int c = v[i];
    v[i] = acc;
    acc += c;
  }
  __syncthreads();
}

__global__ __launch_bounds__(kPrepThreads) void gather_sort_kernel(const int32_t* __restrict__ tok,
                                                                   const int32_t* __restrict__ exp,
                                                                   int B, int E, int T, int N,
                                                                   int ysz, void* __restrict__ y,
                                                                   uint32_t* __restrict__ ws) {
  __shared__ int cnt[kMaxIndexedExperts + 1];
  __shared__ int part[kPrepThreads];
  __shared__ int first_bad;
  for (int e = threadIdx.x; e <= E; e += kPrepThreads) cnt[e] = 0;
  if (threadIdx.x == 0) first_bad = B;
  __syncthreads();
  int mine = B;
  // Expert and token ids of kPrepRun rows per thread, loaded before any is used (one
  // memory latency per pass); with one pass they stay in registers for the second loop.
  int ev[kPrepRun], tv[kPrepRun];
  // Unconditional loads (rows past the end re-read the last one and are not used), the
  // token test outside the unrolled loop: a load under a condition would be waited for
  // where the paths join.
  auto load_ids = [&](int base) {
#pragma unroll
    for (int k = 0; k < kPrepRun; ++k) ev[k] = exp[min(base + (int)threadIdx.x + k * kPrepThreads, B - 1)];
    if (tok) {
#pragma unroll
      for (int k = 0; k < kPrepRun; ++k) tv[k] = tok[min(base + (int)threadIdx.x + k * kPrepThreads, B - 1)];
    } else {
#pragma unroll
      for (int k = 0; k < kPrepRun; ++k) tv[k] = base + (int)threadIdx.x + k * kPrepThreads;
    }
  };
  const bool one_pass = B <= kPrepThreads * kPrepRun;
  for (int base = 0; base < B; base += kPrepThreads * kPrepRun) {
    load_ids(base);
#pragma unroll
    for (int k = 0; k < kPrepRun; ++k) {
      const int r = base + (int)threadIdx.x + k * kPrepThreads;
      if (r >= B) break;
      const int e = ev[k], t = tv[k];
      const bool ok = e >= 0 && e < E && t >= 0 && t < T;
      atomicAdd(&cnt[ok ? e : E], 1);
      if (!ok) mine = min(mine, r);
    }
  }
  if (mine < B) atomicMin(&first_bad, mine);
  __syncthreads();
  block_exclusive_scan(cnt, E + 1, part);  // cnt[e] = first slot of expert e
  int32_t* off = reinterpret_cast<int32_t*>(ws + 1);
  int32_t* perm = reinterpret_cast<int32_t*>(ws + 2 + E);
  for (int e = threadIdx.x; e <= E; e += kPrepThreads) off[e] = cnt[e];
  __syncthreads();
  for (int base = 0; base < B; base += kPrepThreads * kPrepRun) {
    if (!one_pass) load_ids(base);
#pragma unroll
    for (int k = 0; k < kPrepRun; ++k) {
      const int r = base + (int)threadIdx.x + k * kPrepThreads;
      if (r >= B) break;
      const int e = ev[k], t = tv[k];
      const bool ok = e >= 0 && e < E && t >= 0 && t < T;
      perm[atomicAdd(&cnt[ok ? e : E], 1)] = r;
      if (!ok) {
        for (int n = 0; n < N; ++n) {
          if (ysz == 4)
            static_cast<uint32_t*>(y)[(int64_t)r * N + n] = 0u;
          else
            static_cast<uint16_t*>(y)[(int64_t)r * N + n] = 0;
        }
      }
    }
  }
  if (threadIdx.x == 0) ws[0] = first_bad < B ? (uint32_t)first_bad + 1u : 0u;
}

template <typename T>
struct Tile {
  using type = T;
};

// Calls f(Tile<U>{}, r0, rows) over the rows [r_begin, r_end) of one expert: once with a
// tile of 32 or 64 rows when that holds them all and is smaller than T (the MFMAs then
// skip the padding of a short expert), else with T over as many row tiles as the rows
// need, LDS reused between them. The choice is uniform across the workgroup. With
// about 36 rows per expert, a quarter of the experts have 32 rows or fewer: MoE up
// 54.1 -> 52.6 us, down 59.2 -> 57.9, indexed form 55.2 -> 53.8 and 60.8 -> 59.7 (one
// box, same session). Results are bit-identical: a row block's sums do not depend on
// the tile's height.
template <typename T, typename F>
__device__ __forceinline__ void over_expert_rows(int r_begin, int r_end, F&& f) {
  const int n = r_end - r_begin;
  if constexpr (T::BM > 32) {
    static_assert(T::template WithMB<1>::LDS_BYTES <= T::LDS_BYTES, "LDS of the shorter tile");
    if (n <= 32) {
      f(Tile<typename T::template WithMB<1>>{}, r_begin, n);
      return;
    }
  }
  if constexpr (T::BM > 64) {
    static_assert(T::template WithMB<2>::LDS_BYTES <= T::LDS_BYTES, "LDS of the shorter tile");
    if (n <= 64) {
      f(Tile<typename T::template WithMB<2>>{}, r_begin, n);
      return;
    }
  }
  for (int r0 = r_begin; r0 < r_end; r0 += T::BM) {
    if (r0 > r_begin) __syncthreads();  // LDS is reused by the next row block
    f(Tile<T>{}, r0, min(T::BM, r_end - r0));
  }
}

struct GatherParams {
  const uint16_t* x;
  const uint32_t* w;
  const uint16_t* s;
  const uint16_t* b;
  void* y;
  const uint32_t* ws;
  const int32_t* tok;  // indexed form: token per output row (or null)
  int B, N, K, E, T;
  int group;
  int tiles_n;
  int out_f32;
};

template <int BITS, typename T>
__global__ __launch_bounds__(T::THREADS) void gather_qmm_kernel(GatherParams p) {
  __shared__ __attribute__((aligned(16))) char lds[T::LDS_BYTES];
  // Consecutive logical ids (all column blocks of one expert) share an XCD, so the
  // expert's activation rows are fetched into one L2.
  const int L = xcd_remap(blockIdx.x, p.E * p.tiles_n);
  const int e = L / p.tiles_n;
  const int tn = L % p.tiles_n;
  const int n0 = tn * T::BN;
  const size_t ysz = p.out_f32 ? 4 : 2;

  if (p.ws[0] != 0u) {
    // Precondition violated: every row of y becomes zero. Workgroup (e, tn) clears
    // rows [e*per, (e+1)*per) of its column block; together they cover all of y.
    const int per = (p.B + p.E - 1) / p.E;
    const int r0 = e * per;
    const int r1 = min(p.B, r0 + per);
    const int cols = min(T::BN, p.N - n0);
    for (int i = threadIdx.x; i < (r1 > r0 ? (r1 - r0) * cols : 0); i += T::THREADS) {
      const int64_t o = (int64_t)(r0 + i / cols) * p.N + n0 + i % cols;
      if (p.out_f32)
        static_cast<float*>(p.y)[o] = 0.f;
      else
        static_cast<uint16_t*>(p.y)[o] = 0;
    }
    return;
  }
  const int32_t* off = reinterpret_cast<const int32_t*>(p.ws + 1);
  const int r_begin = off[e];
  const int r_end = off[e + 1];
  if (r_begin >= r_end) return;

  const int64_t words = (int64_t)p.K * BITS / 32;
  const int64_t groups = p.K / p.group;
  const uint32_t* we = p.w + (int64_t)e * p.N * words;
  const uint16_t* se = p.s + (int64_t)e * p.N * groups;
  const uint16_t* be = p.b + (int64_t)e * p.N * groups;
  over_expert_rows<T>(r_begin, r_end, [&](auto tile, int r0, int rows) {
    using U = typename decltype(tile)::type;
    U::run(p.x + (int64_t)r0 * p.K, rows, we, se, be, n0, p.N, p.K, p.group,
           static_cast<char*>(p.y) + (size_t)r0 * p.N * ysz, p.out_f32 != 0, lds);
  });
}

// Indexed form: the rows of expert e are perm[off[e] .. off[e+1]); the tile gathers
// their activation rows (through the token index) and scatters its output rows.
template <int BITS, typename T>
__global__ __launch_bounds__(T::THREADS) void gather_qmm_indexed_kernel(GatherParams p) {
  __shared__ __attribute__((aligned(16))) char lds[T::LDS_BYTES];
  const int L = xcd_remap(blockIdx.x, p.E * p.tiles_n);
  const int e = L / p.tiles_n;
  const int tn = L % p.tiles_n;
  const int n0 = tn * T::BN;
  const int32_t* off = reinterpret_cast<const int32_t*>(p.ws + 1);
  const int32_t* perm = reinterpret_cast<const int32_t*>(p.ws + 2 + p.E);
  const int r_begin = off[e];
  const int r_end = off[e + 1];
  if (r_begin >= r_end) return;
  const int64_t words = (int64_t)p.K * BITS / 32;
  const int64_t groups = p.K / p.group;
  const uint32_t* we = p.w + (int64_t)e * p.N * words;
  const uint16_t* se = p.s + (int64_t)e * p.N * groups;
  const uint16_t* be = p.b + (int64_t)e * p.N * groups;
  over_expert_rows<T>(r_begin, r_end, [&](auto tile, int r0, int rows) {
    using U = typename decltype(tile)::type;
    U::run(p.x, rows, we, se, be, n0, p.N, p.K, p.group, p.y, p.out_f32 != 0, lds, perm + r0, p.tok, p.T);
  });
}

template <int BITS, typename T>
hipError_t launch_indexed(GatherParams p, hipStream_t stream) {
  p.tiles_n = (p.N + T::BN - 1) / T::BN;
  hipLaunchKernelGGL((gather_qmm_indexed_kernel<BITS, T>), dim3(p.E * p.tiles_n), dim3(T::THREADS), 0,
                     stream, p);
  launch_log(dim3(p.E * p.tiles_n), dim3(T::THREADS), T::LDS_BYTES, "gather_qmm_indexed_kernel<%d, %s>",
             BITS, T::name());
  return hipGetLastError();
}

template <int BITS, typename T>
hipError_t launch_grouped(GatherParams p, hipStream_t stream) {
  p.tiles_n = (p.N + T::BN - 1) / T::BN;
  hipLaunchKernelGGL((gather_qmm_kernel<BITS, T>), dim3(p.E * p.tiles_n), dim3(T::THREADS), 0,
                     stream, p);
  launch_log(dim3(p.E * p.tiles_n), dim3(T::THREADS), T::LDS_BYTES, "gather_qmm_kernel<%d, %s>", BITS,
             T::name());
  return hipGetLastError();
}

// Scales and biases staged in LDS once per workgroup when the wave's block fits (G <= 48),
// with 4-byte copies when G is even and both arrays 4-byte aligned. Weights in
// 16-row x 64-byte loads (WS; 2-bit codes load their 8 bytes per lane directly), four
// groups ahead: 1-5 % faster than 32 x 32-byte loads three groups ahead on the MoE
// shapes.
template <int BITS, typename T, bool RMAP>
hipError_t launch_form(GatherParams p, hipStream_t stream) {
  if constexpr (RMAP)
    return launch_indexed<BITS, T>(p, stream);
  else
    return launch_grouped<BITS, T>(p, stream);
}

template <int BITS, int MB, bool RMAP>
hipError_t launch_sb(GatherParams p, hipStream_t stream) {
  const int G = p.K / p.group;  // scale values per weight row
  const bool wide = G % 2 == 0 && (reinterpret_cast<uintptr_t>(p.s) & 3) == 0 &&
                    (reinterpret_cast<uintptr_t>(p.b) & 3) == 0;
  if (G <= 12)
    return wide ? launch_form<BITS, MmTile4<BITS, MB, 4, 4, 2, 1, 12, RMAP, BITS != 2>, RMAP>(p, stream)
                : launch_form<BITS, MmTile4<BITS, MB, 4, 4, 2, 2, 12, RMAP, BITS != 2>, RMAP>(p, stream);
  if (G <= 48)
    return wide ? launch_form<BITS, MmTile4<BITS, MB, 4, 4, 2, 1, 48, RMAP, BITS != 2>, RMAP>(p, stream)
                : launch_form<BITS, MmTile4<BITS, MB, 4, 4, 2, 2, 48, RMAP, BITS != 2>, RMAP>(p, stream);
  return launch_form<BITS, MmTile4<BITS, MB, 4, 4, 2, 0, 0, RMAP, BITS != 2>, RMAP>(p, stream);
}

// One row of 4 waves, each with 32 weight rows: every expert's weights are dequantized
// once per column block. Row blocks of 32 per tile from the mean rows per expert, with
// slack for the spread of the routing; experts with more rows loop over row tiles, and
// experts with fewer run a shorter tile (over_expert_rows).
template <int BITS, bool RMAP>
hipError_t launch_tile4(GatherParams p, hipStream_t stream) {
  const int64_t mean = p.E > 0 ? (p.B + p.E - 1) / p.E : p.B;
  const int64_t blocks = (mean + mean / 4 + 31) / 32;
  if (blocks <= 1) return launch_sb<BITS, 1, RMAP>(p, stream);
  if (blocks <= 2) return launch_sb<BITS, 2, RMAP>(p, stream);
  return launch_sb<BITS, 4, RMAP>(p, stream);
}

}  // namespace

size_t gather_workspace_bytes(int64_t E) {
  const size_t raw = (size_t)(E + 2) * sizeof(uint32_t);
  return (raw + 255) / 256 * 256;
}

namespace {

// Workspace of the allocation-free entry point (status word and per-expert offsets),
// one copy per GPU for the life of the process. Every call on a GPU uses that GPU's
// copy, so calls that overlap on one GPU race on it.
constexpr size_t kScratchBytes = 64 * 1024;
static __device__ __align__(256) uint32_t scratch[kScratchBytes / sizeof(uint32_t)];

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch[kMaxScratchDevices];
std::mutex g_scratch_mu;

// Device address of the current GPU's `scratch`, looked up once per device with that
// device current (the host-side name of the array is not a device address).
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

int64_t gather_noalloc_max_experts() {
  return (int64_t)(kScratchBytes / sizeof(uint32_t)) - 2;  // (E + 2) words fit
}

hipError_t launch_gather_qmm_noalloc(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
                                     const uint16_t* biases, const int32_t* expert_idx, void* y,
                                     int64_t B, int64_t N, int64_t K, int64_t E, int bits, int group,
                                     bool out_f32, uint32_t* status, hipStream_t stream) {
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return e;
  return launch_gather_qmm(x, w, scales, biases, expert_idx, y, B, N, K, E, bits, group, out_f32, ws,
                           stream, status);
}

hipError_t launch_gather_qmm(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
                             const uint16_t* biases, const int32_t* expert_idx, void* y,
                             int64_t B, int64_t N, int64_t K, int64_t E, int bits, int group,
                             bool out_f32, void* workspace, hipStream_t stream, uint32_t* status) {
  uint32_t* ws = static_cast<uint32_t*>(workspace);
  hipLaunchKernelGGL(gather_prepare_kernel, dim3(1), dim3(kPrepThreads), 0, stream, expert_idx,
                     (int)B, (int)E, ws, status);
  launch_log(dim3(1), dim3(kPrepThreads), sizeof(int), "gather_prepare_kernel");
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  GatherParams p;
  p.x = x;
  p.w = w;
  p.s = scales;
  p.b = biases;
  p.y = y;
  p.ws = ws;
  p.tok = nullptr;
  p.B = (int)B;
  p.N = (int)N;
  p.K = (int)K;
  p.E = (int)E;
  p.T = (int)B;
  p.group = group;
  p.tiles_n = 0;
  p.out_f32 = out_f32 ? 1 : 0;
  return bits == 4 ? launch_tile4<4, false>(p, stream)
       : bits == 2 ? launch_tile4<2, false>(p, stream)
                   : launch_tile4<8, false>(p, stream);
}

size_t gather_indexed_workspace_bytes(int64_t B, int64_t E) {
  const size_t raw = (size_t)(E + 2 + B) * sizeof(uint32_t);
  return (raw + 255) / 256 * 256;
}

int64_t gather_indexed_max_experts() { return kMaxIndexedExperts; }

hipError_t launch_gather_sort(const int32_t* token_idx, const int32_t* expert_idx, int64_t B,
                              int64_t E, int64_t T, int64_t N, int ysz, void* y, void* workspace,
                              hipStream_t stream) {
  hipLaunchKernelGGL(gather_sort_kernel, dim3(1), dim3(kPrepThreads), 0, stream, token_idx,
                     expert_idx, (int)B, (int)E, (int)T, (int)N, ysz, y,
                     static_cast<uint32_t*>(workspace));
  launch_log(dim3(1), dim3(kPrepThreads), (kMaxIndexedExperts + 1 + kPrepThreads + 1) * sizeof(int),
             "gather_sort_kernel");
  return hipGetLastError();
}

hipError_t launch_gather_qmm_indexed(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
                                     const uint16_t* biases, const int32_t* token_idx,
                                     const int32_t* expert_idx, void* y, int64_t B, int64_t N,
                                     int64_t K, int64_t E, int64_t T, int bits, int group,
                                     bool out_f32, void* workspace, hipStream_t stream) {
  uint32_t* ws = static_cast<uint32_t*>(workspace);
  hipError_t err = launch_gather_sort(token_idx, expert_idx, B, E, T, N, out_f32 ? 4 : 2, y, workspace,
                                      stream);
  if (err != hipSuccess) return err;
  GatherParams p;
  p.x = x;
  p.w = w;
  p.s = scales;
  p.b = biases;
  p.y = y;
  p.ws = ws;
  p.tok = token_idx;
  p.B = (int)B;
  p.N = (int)N;
  p.K = (int)K;
  p.E = (int)E;
  p.T = (int)T;
  p.group = group;
  p.tiles_n = 0;
  p.out_f32 = out_f32 ? 1 : 0;
  return bits == 4 ? launch_tile4<4, true>(p, stream)
       : bits == 2 ? launch_tile4<2, true>(p, stream)
                   : launch_tile4<8, true>(p, stream);
}

}  // namespace bitmm
