// Dense prefill GEMM on the matrix cores (M >= 8): y[M, N] = x[M, K] * dequant(w)^T.
// The epic's kernel table puts the prefill quantized GEMM at 82% of GPU time; the
// tile itself lives in mfma_tile4.hpp.
#include "kernels.hpp"
#include "mfma_tile4.hpp"

namespace bitmm {
namespace {

struct QmmParams {
  const uint16_t* x;
  const uint32_t* w;
  const uint16_t* s;
  const uint16_t* b;
  void* y;
  int M, N, K;
  int group;
  int tiles_m, tiles_n;
  int out_f32;
};

template <typename T>
__global__ __launch_bounds__(T::THREADS) void qmm_mfma_kernel(QmmParams p) {
  __shared__ __attribute__((aligned(16))) char lds[T::LDS_BYTES];
  const int total = p.tiles_m * p.tiles_n;
  // Logical tiles are ordered M-fastest, so the M tiles that share one weight column
  // block run on one XCD and read its codes from that XCD's L2 instead of HBM.
  const int L = xcd_remap(blockIdx.x, total);
  const int tm = L % p.tiles_m;
  const int tn = L / p.tiles_m;
  const int m0 = tm * T::BM;
  const int rows = min(T::BM, p.M - m0);
  const size_t ysz = p.out_f32 ? 4 : 2;
  T::run(p.x + (int64_t)m0 * p.K, rows, p.w, p.s, p.b, tn * T::BN, p.N, p.K, p.group,
         static_cast<char*>(p.y) + (size_t)m0 * p.N * ysz, p.out_f32 != 0, lds);
}

template <typename T>
hipError_t launch_tiles(QmmParams p, hipStream_t stream) {
  p.tiles_m = (p.M + T::BM - 1) / T::BM;
  p.tiles_n = (p.N + T::BN - 1) / T::BN;
  hipLaunchKernelGGL((qmm_mfma_kernel<T>), dim3(p.tiles_m * p.tiles_n), dim3(T::THREADS), 0,
                     stream, p);
  launch_log(dim3(p.tiles_m * p.tiles_n), dim3(T::THREADS), T::LDS_BYTES, "qmm_mfma_kernel<%s>", T::name());
  return hipGetLastError();
}

// 32x32x16 tile: one row of 4 waves, each with 32 weight rows and all the tile's rows
// (blocks of 32, at most 320 rows: three activation buffers fit in LDS). When the groups
// fit (G <= 80, G even, 4-byte aligned scale and bias arrays), each wave's scales and
// biases are staged in LDS once (4-byte copies of its contiguous block) instead of
// being fetched per group: at M = 600, K = 5120 that is the difference between 110 and
// 92 us. At 320 rows the activation buffers and the staging area fill the 160 KB.
// Weights come in 16-row x 64-byte loads (WS), four groups ahead (93 against 95 us).
template <int BITS, int MB>
hipError_t launch_mb(QmmParams p, hipStream_t stream) {
  const int G = p.K / p.group;  // scale values per weight row
  const bool stage = G <= 80 && G % 2 == 0 && (reinterpret_cast<uintptr_t>(p.s) & 3) == 0 &&
                     (reinterpret_cast<uintptr_t>(p.b) & 3) == 0;
  return stage ? launch_tiles<MmTile4<BITS, MB, 4, 4, 2, 1, 80, false, BITS != 2>>(p, stream)
               : launch_tiles<MmTile4<BITS, MB, 4, 4, 2, 0, 0, false, BITS != 2>>(p, stream);
}

// Row blocks per tile. Every tile reads all of K, so the choice trades the tile's own
// speed (fewer rows: shorter loop bodies) against how many tiles the grid needs and
// how many rounds of one tile per CU they take. Timed on the device at K = 5120, one
// tile per CU, a tile of MB row blocks takes about (MB + 5.5) units (MB = 2: 36.5 us,
// 4: 44, 6: 53, 8: 64, 10: 76); the grid's time is its rounds times that. The choice
// minimises it, larger tiles first on ties (fewer re-reads of the weights). For each
// candidate the row blocks are spread evenly over its number of row tiles. Measured
// against one fixed choice: M = 600, K = 13824, N = 5120 (40 column tiles) 219 -> 139 us
// (MB 10 -> 4), M = 600, N = 2048 76 -> 36.5 us (10 -> 2), M = 128, N = 13824 44 -> 38.5
// us (4 -> 2); M = 600, N = 13824 keeps MB = 10 (85 us; 6 gives 110, 8 gives 128).
int pick_row_blocks(int64_t M, int64_t N, int64_t cus) {
  static constexpr int kMB[] = {10, 8, 6, 4, 2, 1};
  const int64_t blocks = (M + 31) / 32;
  const int64_t tiles_n = (N + 127) / 128;
  int best = 10;
  int64_t best_cost = -1;
  for (const int mb : kMB) {
    const int64_t tiles_m = (blocks + mb - 1) / mb;
    const int64_t per = (blocks + tiles_m - 1) / tiles_m;  // row blocks of the fullest tile
    int used = 10;
    for (const int c : kMB)
      if (c >= per) used = c;  // the smallest tile that holds them
    const int64_t rounds = (tiles_m * tiles_n + cus - 1) / cus;
    const int64_t cost = rounds * (2 * used + 11);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = used;
    }
  }
  return best;
}

template <int BITS>
hipError_t launch_tile4(QmmParams p, hipStream_t stream) {
  switch (pick_row_blocks(p.M, p.N, device_compute_units())) {
    case 1: return launch_mb<BITS, 1>(p, stream);
    case 2: return launch_mb<BITS, 2>(p, stream);
    case 4: return launch_mb<BITS, 4>(p, stream);
    case 6: return launch_mb<BITS, 6>(p, stream);
    case 8: return launch_mb<BITS, 8>(p, stream);
    default: return launch_mb<BITS, 10>(p, stream);
  }
}

}  // namespace

hipError_t launch_qmm_mfma(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
                           const uint16_t* biases, void* y, int64_t M, int64_t N, int64_t K,
                           int bits, int group, bool out_f32, hipStream_t stream) {
  QmmParams p;
  p.x = x;
  p.w = w;
  p.s = scales;
  p.b = biases;
  p.y = y;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.group = group;
  p.out_f32 = out_f32 ? 1 : 0;
  p.tiles_m = p.tiles_n = 0;
  return bits == 4 ? launch_tile4<4>(p, stream)
       : bits == 2 ? launch_tile4<2>(p, stream)
                   : launch_tile4<8>(p, stream);
}

}  // namespace bitmm
