// 4-bit instantiations of the small-M GEMV on the matrix cores.
#include "qmv_mfma.hpp"

namespace bitmm {
template hipError_t qmv_mfma_detail::launch_bits<4>(const qmv_mfma_detail::Params&, int, hipStream_t);
}  // namespace bitmm
