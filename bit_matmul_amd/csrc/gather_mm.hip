// Dense grouped product for non-quantized MoE layers (gather_mm): y[r, :] = x[t_r, :] *
// W[e_r]^T over bf16 or binary16 operands. PR #1562 names this path: every
// non-quantized MoE checkpoint reaches the grouped GEMM through
// SwitchLinear::Regular::forward, the same scheduler as the quantized GatherQMM without
// its dequantization, and the PR's tests check it in both operand layouts.
//
// Two kernels on the caller's stream: the indexed gather's counting sort (rows grouped
// by expert in the workspace, rows with out-of-range ids zeroed), then one workgroup per
// (expert, 128-column block) running the dense tile over the expert's rows, 32 MB at a
// time.
#include "dense_tile.hpp"
#include "kernels.hpp"

namespace bitmm {
namespace {

struct GmmParams {
  const uint16_t* x;
  const uint16_t* w;
  void* y;
  const uint32_t* ws;
  const int32_t* tok;
  int B, N, K, E, T;
  int tiles_n;
  int otype;
};

template <typename Tile>
__global__ __launch_bounds__(Tile::THREADS) void gather_mm_kernel(GmmParams p) {
  __shared__ __attribute__((aligned(16))) char lds[Tile::LDS_BYTES];
  // All column blocks of one expert on one XCD: its activation rows meet in one L2.
  const int L = xcd_remap(blockIdx.x, p.E * p.tiles_n);
  const int e = L / p.tiles_n;
  const int tn = L % p.tiles_n;
  const int32_t* off = reinterpret_cast<const int32_t*>(p.ws + 1);
  const int32_t* perm = reinterpret_cast<const int32_t*>(p.ws + 2 + p.E);
  const int r_begin = off[e];
  const int r_end = off[e + 1];
  if (r_begin >= r_end) return;
  const uint16_t* we = p.w + (int64_t)e * p.N * p.K;
  for (int r0 = r_begin; r0 < r_end; r0 += Tile::BM) {
    if (r0 > r_begin) __syncthreads();  // LDS is reused by the next row block
    Tile::run(p.x, p.T, perm + r0, p.tok, min(Tile::BM, r_end - r0), we, tn * Tile::BN, p.N, p.K,
              p.y, p.otype, lds);
  }
}

template <typename Tile>
hipError_t launch_tiles(GmmParams p, hipStream_t stream) {
  p.tiles_n = (p.N + Tile::BN - 1) / Tile::BN;
  hipLaunchKernelGGL((gather_mm_kernel<Tile>), dim3(p.E * p.tiles_n), dim3(Tile::THREADS), 0, stream,
                     p);
  launch_log(dim3(p.E * p.tiles_n), dim3(Tile::THREADS), Tile::LDS_BYTES, "gather_mm_kernel<%s>", Tile::name());
  return hipGetLastError();
}

// Stage depth. 64-k stages (72 KB of LDS at two row blocks) let two workgroups share a
// CU, so one's start-up and epilogue overlap the other's stream; 128-k stages keep the
// 256-byte row copies of [N, K] storage (64-k stages copy 8 rows x 128 bytes, which
// streams slower) but allow one workgroup per CU. Measured on the MoE shapes
// (bf16, 128 experts, ~36 rows each): [N, K] K = 2816: 109 us at 128-k stages, 115 at
// 64; K = 704 (six stages per tile): 133 against 113; [K, N] (256-byte k-rows either
// way): 106 / 100 and 132 / 115.
template <int DT, int LAYOUT, int MB>
hipError_t launch_ks(GmmParams p, hipStream_t stream) {
  if (LAYOUT == 0 && p.K >= 2048) return launch_tiles<MmTileD<DT, LAYOUT, MB, 128, 3>>(p, stream);
  return launch_tiles<MmTileD<DT, LAYOUT, MB, 64, 3>>(p, stream);
}

// Row blocks per tile from the mean rows per expert, with slack for the routing spread:
// one 32-row block up to ~25 rows, else two (experts with more loop over row tiles).
template <int DT, int LAYOUT>
hipError_t launch_mb(GmmParams p, hipStream_t stream) {
  const int64_t mean = (p.B + p.E - 1) / p.E;
  if (mean + mean / 4 <= 32) return launch_ks<DT, LAYOUT, 1>(p, stream);
  return launch_ks<DT, LAYOUT, 2>(p, stream);
}

}  // namespace

hipError_t launch_gather_mm(const uint16_t* x, const uint16_t* w, const int32_t* token_idx,
                            const int32_t* expert_idx, void* y, int64_t B, int64_t N, int64_t K,
                            int64_t E, int64_t T, int dtype, int layout, int otype,
                            void* workspace, hipStream_t stream) {
  hipError_t err = launch_gather_sort(token_idx, expert_idx, B, E, T, N, otype == kOutF32 ? 4 : 2, y,
                                      workspace, stream);
  if (err != hipSuccess) return err;
  GmmParams p;
  p.x = x;
  p.w = w;
  p.y = y;
  p.ws = static_cast<const uint32_t*>(workspace);
  p.tok = token_idx;
  p.B = (int)B;
  p.N = (int)N;
  p.K = (int)K;
  p.E = (int)E;
  p.T = (int)T;
  p.tiles_n = 0;
  p.otype = otype;
  if (dtype == 0)
    return layout == 0 ? launch_mb<0, 0>(p, stream) : launch_mb<0, 1>(p, stream);
  return layout == 0 ? launch_mb<1, 0>(p, stream) : launch_mb<1, 1>(p, stream);
}

}  // namespace bitmm
