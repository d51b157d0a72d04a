// Decode-stage GEMV: host dispatch (see gemv_kernel.hpp for the kernel).
#include "gemv_kernel.hpp"

namespace w4a8 {
namespace gemv_detail {

W4A8_GEMV_INSTANTIATE(kGemvOut, 1, false)

#define W4A8_GEMV_EXTERN(MODE, MR, NORM)                                                                  \
  extern template int launch_rows_mr<MODE, MR, NORM>(const GemvArgs&, Scratch*, unsigned long long*, \
                                                     hipStream_t);
W4A8_GEMV_EXTERN(kGemvOut, 2, false)
W4A8_GEMV_EXTERN(kGemvOut, 4, false)
W4A8_GEMV_EXTERN(kGemvOut, 8, false)
W4A8_GEMV_EXTERN(kGemvSums, 1, false)
W4A8_GEMV_EXTERN(kGemvSums, 8, false)
W4A8_GEMV_EXTERN(kGemvArgmax, 1, false)
W4A8_GEMV_EXTERN(kGemvArgmax, 8, false)
W4A8_GEMV_EXTERN(kGemvArgmax, 1, true)
W4A8_GEMV_EXTERN(kGemvCast, 1, true)
W4A8_GEMV_EXTERN(kGemvResid, 1, false)
W4A8_GEMV_EXTERN(kGemvGated, 1, true)
#undef W4A8_GEMV_EXTERN

// Rows r0 .. r0 + rows - 1 of the call.
GemvArgs row_slice(const GemvArgs& a, int r0, int rows) {
  GemvArgs s = a;
  s.M = rows;
  if (a.x) s.x = a.x + static_cast<int64_t>(r0) * a.K;
  if (a.xf) s.xf = a.xf + static_cast<int64_t>(r0) * a.K;
  if (a.out) s.out = a.out + static_cast<int64_t>(r0) * a.N;
  if (a.sums) s.sums = a.sums + static_cast<int64_t>(r0) * a.N * (a.K / kBlock);
  if (a.logits) s.logits = a.logits + static_cast<int64_t>(r0) * a.N;
  if (a.argmax) s.argmax = a.argmax + r0;
  if (a.resid) s.resid = a.resid + static_cast<int64_t>(r0) * a.N;
  return s;
}

template <int MODE>
int launch_rows(const GemvArgs& a, int r0, int rows, Scratch* sc, hipStream_t stream) {
  const GemvArgs s = row_slice(a, r0, rows);
  unsigned long long* slots = sc->slots + (MODE == kGemvArgmax ? r0 * kArgmaxSpread : 0);
  if (rows == 1) return launch_rows_mr<MODE, 1, false>(s, sc, slots, stream);
  if constexpr (MODE == kGemvOut) {
    if (rows == 2) return launch_rows_mr<MODE, 2, false>(s, sc, slots, stream);
    if (rows <= 4) return launch_rows_mr<MODE, 4, false>(s, sc, slots, stream);
  }
  return launch_rows_mr<MODE, 8, false>(s, sc, slots, stream);
}

}  // namespace gemv_detail

using gemv_detail::kRowsMax;
using gemv_detail::launch_rows;

size_t gemv_scratch_bytes(int, int, int) { return 0; }

namespace {
// One wave per row: the maximum key over the row's slots gives the index
// (lowest column among equal values); the slots are cleared for the next
// launch.  Device-scope accesses: the slots were written by device-scope
// atomics of the previous kernel.
__global__ __launch_bounds__(64) void argmax_finalize_kernel(unsigned long long* __restrict__ slots,
                                                             int32_t* __restrict__ argmax_out) {
  static_assert(kArgmaxSpread == 64, "one lane per slot");
  const int m = blockIdx.x;
  unsigned long long* row = slots + m * kArgmaxSpread;
  unsigned long long key = __hip_atomic_load(&row[threadIdx.x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const unsigned long long o = __shfl_xor(key, off);
    key = o > key ? o : key;
  }
  __hip_atomic_store(&row[threadIdx.x], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (threadIdx.x == 0) argmax_out[m] = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(key & 0xFFFFFFFFull));
}

int launch_argmax_finalize(Scratch* sc, int M, int32_t* argmax, hipStream_t stream) {
  hipLaunchKernelGGL(argmax_finalize_kernel, dim3(M), dim3(64), 0, stream, sc->slots, argmax);
  W4A8_HIP(hipGetLastError());
  return W4A8_OK;
}
}  // namespace

bool gemv_fused_supported(int mode, bool norm, int K, int N) {
  if (mode < kGemvCast && !(mode == kGemvArgmax && norm)) return false;
  if (!norm) return true;
  // The normalising prologue needs every block of the row in one chunk.
  return gemv_detail::chunk_blocks(gemv_detail::pick_plan(K, N, true)) >= K / kBlock;
}

int launch_gemv(const GemvArgs& a, int mode, Scratch* sc, hipStream_t stream) {
  int rc = W4A8_OK;
  if (mode == kGemvArgmax && (!sc->slots || a.M > kMaxArgmaxRows))
    return hip_fail(hipErrorInvalidValue, "gemv: argmax needs the library's argmax slots");
  if (mode >= kGemvCast || a.xf) {
    // Fused decoder-layer kernels: one token row.
    if (a.M != 1 || !gemv_fused_supported(mode, a.xf != nullptr, a.K, a.N))
      return hip_fail(hipErrorInvalidValue, "gemv: fused launch outside its shapes");
    using gemv_detail::launch_rows_mr;
    if (mode == kGemvCast) return launch_rows_mr<kGemvCast, 1, true>(a, sc, sc->slots, stream);
    if (mode == kGemvResid) return launch_rows_mr<kGemvResid, 1, false>(a, sc, sc->slots, stream);
    if (mode == kGemvGated) return launch_rows_mr<kGemvGated, 1, true>(a, sc, sc->slots, stream);
    rc = launch_rows_mr<kGemvArgmax, 1, true>(a, sc, sc->slots, stream);
    if (rc != W4A8_OK) return rc;
    return launch_argmax_finalize(sc, 1, a.argmax, stream);
  }
  for (int r0 = 0; r0 < a.M; r0 += kRowsMax) {
    const int rows = a.M - r0 < kRowsMax ? a.M - r0 : kRowsMax;
    if (mode == kGemvOut) rc = launch_rows<kGemvOut>(a, r0, rows, sc, stream);
    else if (mode == kGemvSums) rc = launch_rows<kGemvSums>(a, r0, rows, sc, stream);
    else rc = launch_rows<kGemvArgmax>(a, r0, rows, sc, stream);
    if (rc != W4A8_OK) return rc;
  }
  if (mode == kGemvArgmax) return launch_argmax_finalize(sc, a.M, a.argmax, stream);
  return W4A8_OK;
}

}  // namespace w4a8
