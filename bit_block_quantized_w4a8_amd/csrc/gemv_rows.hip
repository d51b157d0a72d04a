// Decode-stage GEMV instantiations: 2, 4 and 8 token rows.
#include "gemv_kernel.hpp"

namespace w4a8 {
namespace gemv_detail {
W4A8_GEMV_INSTANTIATE(kGemvOut, 2, false)
W4A8_GEMV_INSTANTIATE(kGemvOut, 4, false)
W4A8_GEMV_INSTANTIATE(kGemvOut, 8, false)
}  // namespace gemv_detail
}  // namespace w4a8
