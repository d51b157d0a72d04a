// Decode-stage GEMV instantiations: 2, 4 and 8 token rows.
#include "gemv_kernel.hpp"

namespace w4a8 {
namespace gemv_detail {
W4A8_GEMV_INSTANTIATE(0, 2)
W4A8_GEMV_INSTANTIATE(0, 4)
W4A8_GEMV_INSTANTIATE(0, 8)
}  // namespace gemv_detail
}  // namespace w4a8
