// Host side of the GEMV / small-M path. Three kernel forms:
//   qmv_dma_kernel (qmv_dma.hpp): one activation row, K up to 5 chunks per lane
//     (K <= 10240 at 4 bits, <= 5120 at 8 bits, <= 20480 at 2 bits), the decode GEMV;
//   qmv_split_kernel (qmv_split.hpp): up to 8 activation rows with K split across the
//     waves of a workgroup (K <= 16384 at 4 bits and 8192 at 8 bits for up to 3 rows,
//     half that from 4 rows; 2 bits: up to 3 rows, K <= 16384), the small-M prefill tail;
//   qmv_mfma_kernel (qmv_mfma.hpp): 2 to 8 activation rows on the matrix cores (K <= 16384
//     at 4 bits, 8192 at 8, 32768 at 2; more rows in launches of 8), the small-M prefill
//     tail;
//   qmv_kernel (qmv_impl.hpp): up to 8 activation rows per launch, any K (several
//     passes over K when a row does not fit), for what the others do not take (2-bit
//     codes with K past the split kernel's range: four rows per launch).
#include "kernels.hpp"
#include "qmv_dma.hpp"
#include "qmv_impl.hpp"
#include "qmv_mfma.hpp"
#include "qmv_split.hpp"

namespace bitmm {

namespace {

// One launch sequence over M activation rows (a dense call), or over the gathered rows
// of `bt` with one activation row each (M = 1).
hipError_t launch_rows(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
                       const uint16_t* biases, void* y, int64_t M, int64_t N, int64_t K, int bits,
                       int group, bool out_f32, const GemvBatch& bt, hipStream_t stream) {
  const int64_t nch = K * bits / 128;  // 16-byte code chunks per weight row
  const size_t ysz = out_f32 ? 4 : 2;
  // 2-bit codes: the decode kernel for one row, the split-K kernel for up to 3 rows (more
  // rows in launches of 3), else the general kernel (rows four at a time).
  if (M == 1 && qmv_dma_detail::pick_lanes(nch) != 0) {
    qmv_dma_detail::Params dp;
    dp.x = x;
    dp.w = w;
    dp.s = scales;
    dp.b = biases;
    dp.y = y;
    dp.N = (int)N;
    dp.K = (int)K;
    dp.gshift = group_shift(group);
    dp.out_f32 = out_f32 ? 1 : 0;
    dp.steps_per_wave = dp.total_steps = 0;
    dp.bt = bt;
    return bits == 4   ? qmv_dma_detail::launch_bits<4>(dp, device_compute_units(), 0, stream)
           : bits == 2 ? qmv_dma_detail::launch_bits<2>(dp, device_compute_units(), 0, stream)
                       : qmv_dma_detail::launch_bits<8>(dp, device_compute_units(), 0, stream);
  }
  // Dense calls with several rows: the matrix-core GEMV, eight rows per launch.
  if (bt.exp == nullptr && M >= 2 && qmv_mfma_detail::fits(K, bits, M < 8 ? M : 8)) {
    for (int64_t m0 = 0; m0 < M; m0 += 8) {
      qmv_mfma_detail::Params mp;
      mp.x = x + m0 * K;
      mp.w = w;
      mp.s = scales;
      mp.b = biases;
      mp.y = static_cast<char*>(y) + (size_t)(m0 * N) * ysz;
      mp.M = (int)(M - m0 < 8 ? M - m0 : 8);
      mp.N = (int)N;
      mp.K = (int)K;
      mp.gshift = group_shift(group);
      mp.out_f32 = out_f32 ? 1 : 0;
      mp.mask = 0x000F000Fu;
      mp.magic = 0x43004300u;
      const hipError_t e = bits == 4   ? qmv_mfma_detail::launch_bits<4>(mp, device_compute_units(), stream)
                           : bits == 2 ? qmv_mfma_detail::launch_bits<2>(mp, device_compute_units(), stream)
                                       : qmv_mfma_detail::launch_bits<8>(mp, device_compute_units(), stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  if (M <= 8 && qmv_split_detail::fits(K, bits, M)) {
    qmv_split_detail::Params sp;
    sp.x = x;
    sp.w = w;
    sp.s = scales;
    sp.b = biases;
    sp.y = y;
    sp.N = (int)N;
    sp.K = (int)K;
    sp.gshift = group_shift(group);
    sp.out_f32 = out_f32 ? 1 : 0;
    sp.bt = bt;
    return bits == 4   ? qmv_split_detail::launch_bits<4>(sp, (int)M, stream)
           : bits == 2 ? qmv_split_detail::launch_bits<2>(sp, (int)M, stream)
                       : qmv_split_detail::launch_bits<8>(sp, (int)M, stream);
  }
  // 2-bit codes beyond 3 rows: launches of up to 3 rows on the kernels above (the split
  // kernel takes 3 rows in about 40 % of the time the general kernel needs for 4).
  if (bits == 2 && M > 3 && qmv_split_detail::fits(K, 2, 3)) {
    for (int64_t m0 = 0; m0 < M; m0 += 3) {
      const int64_t mr = M - m0 < 3 ? M - m0 : 3;
      const hipError_t e = launch_rows(x + m0 * K, w, scales, biases, static_cast<char*>(y) + (size_t)(m0 * N) * ysz,
                                       mr, N, K, bits, group, out_f32, bt, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const int rows_per_launch = bits == 2 ? 4 : 8;
  for (int64_t m0 = 0; m0 < M; m0 += rows_per_launch) {
    const int mr = (int)(M - m0 < rows_per_launch ? M - m0 : rows_per_launch);
    // Chunks per lane per pass over K: as few passes as possible, with at most
    // 4 chunks, and at most 12 chunk-rows of activations held per lane (at 2 bits,
    // where a chunk has twice the activations, 2 chunks for one row and 1 beyond).
    const int64_t cap = bits == 2 ? (mr == 1 ? 2 : 1) : (mr <= 3 ? 4 : (12 / mr > 0 ? 12 / mr : 1));
    const int64_t passes = (nch + cap * kWave - 1) / (cap * kWave);
    const int cpl = (int)((nch + passes * kWave - 1) / (passes * kWave));
    qmv_detail::QmvParams p;
    p.x = x + m0 * K;
    p.w = w;
    p.s = scales;
    p.b = biases;
    p.y = static_cast<char*>(y) + (size_t)(m0 * N) * ysz;
    p.N = (int)N;
    p.K = (int)K;
    p.gshift = group_shift(group);
    p.out_f32 = out_f32 ? 1 : 0;
    p.bt = bt;
    const hipError_t e = bits == 4   ? qmv_detail::launch_bits<4>(p, mr, cpl, stream)
                         : bits == 2 ? qmv_detail::launch_bits<2>(p, mr, cpl, stream)
                                     : qmv_detail::launch_bits<8>(p, mr, cpl, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

bool qmv_mfma_takes(int64_t K, int bits, int64_t M) { return qmv_mfma_detail::fits(K, bits, M); }

hipError_t launch_qmv(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
                      const uint16_t* biases, void* y, int64_t M, int64_t N, int64_t K, int bits,
                      int group, bool out_f32, hipStream_t stream) {
  GemvBatch none{};
  return launch_rows(x, w, scales, biases, y, M, N, K, bits, group, out_f32, none, stream);
}

hipError_t launch_gather_qmv(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
                             const uint16_t* biases, const int32_t* token_idx,
                             const int32_t* expert_idx, void* y, int64_t B, int64_t N, int64_t K,
                             int64_t E, int64_t T, int bits, int group, bool out_f32,
                             hipStream_t stream) {
  constexpr int64_t kMaxGridRows = 65535;  // one launch per this many output rows
  GemvBatch bt;
  bt.tok = token_idx;
  bt.exp = expert_idx;
  bt.T = (int)T;
  bt.E = (int)E;
  bt.w_stride = N * K * bits / 32;
  bt.sb_stride = N * (K / group);
  for (int64_t r0 = 0; r0 < B; r0 += kMaxGridRows) {
    bt.row0 = (int)r0;
    bt.rows = (int)(B - r0 < kMaxGridRows ? B - r0 : kMaxGridRows);
    const hipError_t e = launch_rows(x, w, scales, biases, y, 1, N, K, bits, group, out_f32, bt, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace bitmm
