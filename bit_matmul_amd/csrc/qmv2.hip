// 2-bit instantiations of the GEMV / small-M kernel.
#include "qmv_impl.hpp"

namespace bitmm {
template hipError_t qmv_detail::launch_bits<2>(const qmv_detail::QmvParams&, int, int,
                                                hipStream_t);
}  // namespace bitmm
