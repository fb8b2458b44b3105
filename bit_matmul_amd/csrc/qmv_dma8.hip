// 8-bit instantiations of the decode GEMV.
#include "qmv_dma.hpp"

namespace bitmm {
template hipError_t qmv_dma_detail::launch_bits<8>(const qmv_dma_detail::Params&, int, int, hipStream_t);
}  // namespace bitmm
