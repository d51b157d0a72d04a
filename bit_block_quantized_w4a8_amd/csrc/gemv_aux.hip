// Decode-stage GEMV instantiations: integer block-sum export and fused argmax.
#include "gemv_kernel.hpp"

namespace w4a8 {
namespace gemv_detail {
W4A8_GEMV_INSTANTIATE(kGemvSums, 1, false)
W4A8_GEMV_INSTANTIATE(kGemvSums, 8, false)
W4A8_GEMV_INSTANTIATE(kGemvArgmax, 1, false)
W4A8_GEMV_INSTANTIATE(kGemvArgmax, 8, false)
}  // namespace gemv_detail
}  // namespace w4a8
