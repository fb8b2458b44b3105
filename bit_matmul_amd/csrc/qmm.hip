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

template <int BITS>
hipError_t launch_tile4(QmmParams p, hipStream_t stream) {
  const int64_t blocks = (p.M + 31) / 32;
  const int64_t tiles = (blocks + 9) / 10;
  const int64_t per = (blocks + tiles - 1) / tiles;
  if (per <= 1) return launch_mb<BITS, 1>(p, stream);
  if (per <= 2) return launch_mb<BITS, 2>(p, stream);
  if (per <= 4) return launch_mb<BITS, 4>(p, stream);
  if (per <= 6) return launch_mb<BITS, 6>(p, stream);
  if (per <= 8) return launch_mb<BITS, 8>(p, stream);
  return launch_mb<BITS, 10>(p, stream);
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
