// Decode-stage GEMV: host dispatch (see gemv_kernel.hpp for the kernel).
#include "gemv_kernel.hpp"

namespace w4a8 {
namespace gemv_detail {

W4A8_GEMV_INSTANTIATE(0, 1)

extern template int launch_rows_mr<0, 2>(const GemvArgs&, int, int, const uint16_t*, float*, int32_t*, float*,
                                         int32_t*, Scratch*, unsigned long long*, hipStream_t);
extern template int launch_rows_mr<0, 4>(const GemvArgs&, int, int, const uint16_t*, float*, int32_t*, float*,
                                         int32_t*, Scratch*, unsigned long long*, hipStream_t);
extern template int launch_rows_mr<0, 8>(const GemvArgs&, int, int, const uint16_t*, float*, int32_t*, float*,
                                         int32_t*, Scratch*, unsigned long long*, hipStream_t);
extern template int launch_rows_mr<1, 1>(const GemvArgs&, int, int, const uint16_t*, float*, int32_t*, float*,
                                         int32_t*, Scratch*, unsigned long long*, hipStream_t);
extern template int launch_rows_mr<1, 8>(const GemvArgs&, int, int, const uint16_t*, float*, int32_t*, float*,
                                         int32_t*, Scratch*, unsigned long long*, hipStream_t);
extern template int launch_rows_mr<2, 1>(const GemvArgs&, int, int, const uint16_t*, float*, int32_t*, float*,
                                         int32_t*, Scratch*, unsigned long long*, hipStream_t);
extern template int launch_rows_mr<2, 8>(const GemvArgs&, int, int, const uint16_t*, float*, int32_t*, float*,
                                         int32_t*, Scratch*, unsigned long long*, hipStream_t);

template <int MODE>
int launch_rows(const GemvArgs& a, int r0, int rows, Scratch* sc, hipStream_t stream) {
  const int cols = pick_columns(a.N);
  const uint16_t* x = a.x + static_cast<int64_t>(r0) * a.K;
  float* out = a.out ? a.out + static_cast<int64_t>(r0) * a.N : nullptr;
  int32_t* sums = a.sums ? a.sums + static_cast<int64_t>(r0) * a.N * (a.K / kBlock) : nullptr;
  float* logits = a.logits ? a.logits + static_cast<int64_t>(r0) * a.N : nullptr;
  int32_t* am = a.argmax ? a.argmax + r0 : nullptr;
  unsigned long long* slots = sc->slots + (MODE == 2 ? r0 : 0);
  if (rows == 1) return launch_rows_mr<MODE, 1>(a, rows, cols, x, out, sums, logits, am, sc, slots, stream);
  if constexpr (MODE == 0) {
    if (rows == 2) return launch_rows_mr<MODE, 2>(a, rows, cols, x, out, sums, logits, am, sc, slots, stream);
    if (rows <= 4) return launch_rows_mr<MODE, 4>(a, rows, cols, x, out, sums, logits, am, sc, slots, stream);
  }
  return launch_rows_mr<MODE, 8>(a, rows, cols, x, out, sums, logits, am, sc, slots, stream);
}

}  // namespace gemv_detail

using gemv_detail::kRowsMax;
using gemv_detail::launch_rows;

size_t gemv_scratch_bytes(int, int, int) { return 0; }

int launch_gemv(const GemvArgs& a, int mode, hipStream_t stream) {
  Scratch* sc = nullptr;
  int rc = scratch_for(0, &sc);
  if (rc != W4A8_OK) return rc;
  for (int r0 = 0; r0 < a.M; r0 += kRowsMax) {
    const int rows = a.M - r0 < kRowsMax ? a.M - r0 : kRowsMax;
    if (mode == 0) rc = launch_rows<0>(a, r0, rows, sc, stream);
    else if (mode == 1) rc = launch_rows<1>(a, r0, rows, sc, stream);
    else rc = launch_rows<2>(a, r0, rows, sc, stream);
    if (rc != W4A8_OK) return rc;
  }
  return W4A8_OK;
}

}  // namespace w4a8
