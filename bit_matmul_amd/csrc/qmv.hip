// Host side of the GEMV / small-M path (kernel in qmv_impl.hpp).
#include "kernels.hpp"
#include "qmv_impl.hpp"

namespace bitmm {

hipError_t launch_qmv(const uint16_t* x, const uint32_t* w, const uint16_t* scales,
                      const uint16_t* biases, void* y, int64_t M, int64_t N, int64_t K, int bits,
                      bool out_f32, hipStream_t stream) {
  const int64_t cc = 128 / bits;
  const int64_t nch = K / cc;
  // Chunks per lane per pass: the fewest passes over K with at most 4 chunks each.
  const int64_t passes = (nch + 4 * kWave - 1) / (4 * kWave);
  const int cpl = (int)((nch + passes * kWave - 1) / (passes * kWave));
  const size_t ysz = out_f32 ? 4 : 2;
  for (int64_t m0 = 0; m0 < M; m0 += 8) {
    const int mr = (int)(M - m0 < 8 ? M - m0 : 8);
    qmv_detail::QmvParams p;
    p.x = x + m0 * K;
    p.w = w;
    p.s = scales;
    p.b = biases;
    p.y = static_cast<char*>(y) + (size_t)(m0 * N) * ysz;
    p.N = (int)N;
    p.K = (int)K;
    p.out_f32 = out_f32 ? 1 : 0;
    hipError_t e = bits == 4 ? qmv_detail::launch_bits<4>(p, mr, cpl, stream)
                              : qmv_detail::launch_bits<8>(p, mr, cpl, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace bitmm
