// Decode-stage GEMV instantiations of the one-row decoder-layer kernels: the
// normalising prologue (qkv, gate/up and the LM head read the fp32 residual
// stream) and the cast, residual and gated epilogues.
#include "gemv_kernel.hpp"

namespace w4a8 {
namespace gemv_detail {
W4A8_GEMV_INSTANTIATE(kGemvCast, 1, true)
W4A8_GEMV_INSTANTIATE(kGemvResid, 1, false)
W4A8_GEMV_INSTANTIATE(kGemvGated, 1, true)
W4A8_GEMV_INSTANTIATE(kGemvArgmax, 1, true)
}  // namespace gemv_detail
}  // namespace w4a8
