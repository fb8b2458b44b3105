// 2-bit instantiations of the split-K small-M GEMV.
#include "qmv_split.hpp"

namespace bitmm {
template hipError_t qmv_split_detail::launch_bits<2>(const qmv_split_detail::Params&, int, hipStream_t);
}  // namespace bitmm
