// 8-bit instantiations of the matrix-core GEMV / small-M kernel.
#include "qmv_mfma.hpp"

namespace bitmm {
template hipError_t qmv_detail::launch_mfma_bits<8>(const qmv_detail::QmvMfmaParams&, int, int,
                                                     hipStream_t);
}  // namespace bitmm
