// Decode-stage GEMV instantiations: integer block-sum export and fused argmax.
#include "gemv_kernel.hpp"

namespace w4a8 {
namespace gemv_detail {
W4A8_GEMV_INSTANTIATE(1, 1)
W4A8_GEMV_INSTANTIATE(1, 8)
W4A8_GEMV_INSTANTIATE(2, 1)
W4A8_GEMV_INSTANTIATE(2, 8)
}  // namespace gemv_detail
}  // namespace w4a8
