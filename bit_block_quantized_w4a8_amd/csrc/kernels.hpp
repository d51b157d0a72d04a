// Launchers of the W4A8 kernels (host side, C++ linkage, library-internal).
#pragma once

#include "common.hpp"

namespace w4a8 {

int launch_pack(const int8_t* q, const uint16_t* s, int K, int N, uint8_t* packed,
                uint16_t* w_scales, hipStream_t stream);

int launch_quantize_export(const uint16_t* x, int M, int K, int8_t* qx, float* sx,
                           hipStream_t stream);

int launch_quantize_stage(const uint16_t* x, int M, int M_pad, int K, uint8_t* qxs, float* sxs,
                          hipStream_t stream);

// Decode GEMV (int8 dot products, activations quantised in the kernel).
// mode: 0 = scaled output, 1 = integer block sums, 2 = fused argmax (+ optional logits).
struct GemvArgs {
  const uint16_t* x;
  const uint8_t* packed_w;
  const uint16_t* w_scales;
  int M, K, N;
  float* out;            // mode 0
  int32_t* sums;         // mode 1
  float* logits;         // mode 2, may be null
  int32_t* argmax;       // mode 2
};
int launch_gemv(const GemvArgs& a, int mode, hipStream_t stream);
size_t gemv_scratch_bytes(int M, int K, int N);

// Prefill GEMM (int8 MFMA on pre-quantised activations).
// mode: 0 = scaled output, 1 = integer block sums.
struct GemmArgs {
  const uint16_t* x;
  const uint8_t* packed_w;
  const uint16_t* w_scales;
  int M, K, N;
  float* out;            // mode 0
  int32_t* sums;         // mode 1
};
int launch_gemm(const GemmArgs& a, int mode, hipStream_t stream);
size_t gemm_scratch_bytes(int M, int K, int N);

int gemv_max_m();

// Glue of the synthetic decoder layer (layer.hip).
int launch_residual_norm_cast(float* x, const float* d, int64_t ld_d, float alpha, float eps, int M, int H,
                              uint16_t* y, hipStream_t stream);
int launch_cast_rows(const float* src, int64_t ld, int M, int H, uint16_t* dst, hipStream_t stream);
int launch_gated_cast(const float* g, int M, int F, uint16_t* u, hipStream_t stream);

// Byte offsets of a decoder layer's temporaries inside the caller's workspace.
struct LayerWorkspace {
  size_t q, a, o, n, g, u, d, bytes;
};
LayerWorkspace layer_workspace(int M, int H, int n_qkv, int n_gu);

}  // namespace w4a8
