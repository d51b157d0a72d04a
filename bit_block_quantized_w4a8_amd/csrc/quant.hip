// Weight packer and activation quantiser kernels (gfx950).
#include "kernels.hpp"

namespace w4a8 {

// ------------------------------------------------------------------ packer
// One thread per (block b, column n): reads the 32 int4 values of column n in
// block b and writes the 16-byte group packed_w[b][n][0..15] (byte j: element
// 32b+j in the low nibble, element 32b+16+j in the high nibble) and the scale
// w_scales[b][n] = s[n][b].  Off the timed path: weights are packed once.
__global__ __launch_bounds__(256) void pack_kernel(const int8_t* __restrict__ q,
                                                   const uint16_t* __restrict__ s, int K, int N,
                                                   uint8_t* __restrict__ packed,
                                                   uint16_t* __restrict__ w_scales) {
  const int nb = K / kBlock;
  const int64_t total = static_cast<int64_t>(nb) * N;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const int b = static_cast<int>(t / N);
  const int n = static_cast<int>(t % N);
  const int8_t* src = q + static_cast<int64_t>(n) * K + static_cast<int64_t>(b) * kBlock;
  uint32_t words[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = 4 * d + e;
      const uint32_t lo = static_cast<uint32_t>(src[j]) & 0xFu;
      const uint32_t hi = static_cast<uint32_t>(src[j + 16]) & 0xFu;
      w |= (lo | (hi << 4)) << (8 * e);
    }
    words[d] = w;
  }
  *reinterpret_cast<uint4*>(packed + t * kPackedBytes) = make_uint4(words[0], words[1], words[2], words[3]);
  w_scales[t] = s[static_cast<int64_t>(n) * nb + b];
}

int launch_pack(const int8_t* q, const uint16_t* s, int K, int N, uint8_t* packed,
                uint16_t* w_scales, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(K / kBlock) * N;
  const int64_t grid = (total + 255) / 256;
  hipLaunchKernelGGL(pack_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, q, s, K, N,
                     packed, w_scales);
  W4A8_HIP(hipGetLastError());
  return W4A8_OK;
}

// -------------------------------------------------------- quantiser export
// Thread t quantises elements 8g .. 8g+7 of block b of row m, with 4
// consecutive threads per block (K/8 is a multiple of 4, so the groups of 4 are
// lane-aligned and whole groups are in or out of range together).
__global__ __launch_bounds__(256) void quantize_export_kernel(const uint16_t* __restrict__ x, int M,
                                                              int K, int8_t* __restrict__ qx,
                                                              float* __restrict__ sx) {
  const int64_t per_row = K / 8;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= per_row * M) return;
  const int64_t m = t / per_row;
  const int64_t e = t % per_row;  // 8-element group index within the row
  float v[8];
  unpack_half8(*reinterpret_cast<const uint4*>(x + m * K + 8 * e), v);
  float scale;
  const uint2 codes = quantize8_group4(v, &scale);
  *reinterpret_cast<uint2*>(qx + m * K + 8 * e) = codes;
  if ((e & 3) == 0) sx[m * (K / kBlock) + e / 4] = scale;
}

int launch_quantize_export(const uint16_t* x, int M, int K, int8_t* qx, float* sx,
                           hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(M) * (K / 8);
  const int64_t grid = (total + 255) / 256;
  hipLaunchKernelGGL(quantize_export_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream,
                     x, M, K, qx, sx);
  W4A8_HIP(hipGetLastError());
  return W4A8_OK;
}

// ------------------------------------------------------ GEMM pre-pass
// Quantises x [M][K] into the staging layout read by the MFMA GEMM:
//   qxs int8, per block b: [M_pad/32][2][32][16] -- row group (32 rows), lane
//       half h, row within the group, 16 bytes.  Half h of (block b, row m)
//       holds elements 8h .. 8h+7 followed by 16+8h .. 16+8h+7, the order in
//       which the weight nibbles unpack (see gemm.hip), so lane (h, r) of an
//       MFMA operand finds its 16 bytes at ((group * 2 + h) * 32 + r) * 16 and
//       a wave's 64 fragment reads touch 64 consecutive 16-byte slots;
//   sxs [K/32][M_pad] fp32 block scales.
// Rows M .. M_pad-1 are written as zeros (codes and scales).
// A quad of lanes quantises one (row, block); consecutive quads take
// consecutive rows of the same block, so a wave writes whole runs of the
// staging layout.  Group lane g holds elements 8g .. 8g+7, which belong at
// byte 8 * (0, 2, 1, 3)[g] of the row's 32 codes: half (0, 1, 0, 1)[g],
// offset (0, 0, 8, 8)[g].  The grid's x dimension covers the rows (four
// lanes each) and its y dimension the blocks, so no lane divides by a
// runtime size to find its (row, block).
__global__ __launch_bounds__(256) void quantize_stage_kernel(const uint16_t* __restrict__ x, int M,
                                                             int M_pad, int K,
                                                             uint8_t* __restrict__ qxs,
                                                             float* __restrict__ sxs) {
  const int tx = blockIdx.x * blockDim.x + threadIdx.x;
  if (tx >= 4 * M_pad) return;  // whole quads (4 | 256)
  const int g = tx & 3;
  const int64_t m = tx >> 2;
  const int nb = K / kBlock;
  for (int b = blockIdx.y; b < nb; b += gridDim.y) {
    const int64_t e = 4 * static_cast<int64_t>(b) + g;  // 8-element group index within the row
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (m < M) unpack_half8(*reinterpret_cast<const uint4*>(x + m * K + 8 * e), v);
    quantize_to_staging(v, m, e, M_pad, qxs, sxs);
  }
}

int launch_quantize_stage(const uint16_t* x, int M, int M_pad, int K, uint8_t* qxs, float* sxs,
                          hipStream_t stream) {
  const int nb = K / kBlock;
  const dim3 grid((4 * M_pad + 255) / 256, nb < 65535 ? nb : 65535);
  hipLaunchKernelGGL(quantize_stage_kernel, grid, dim3(256), 0, stream, x, M, M_pad, K, qxs, sxs);
  W4A8_HIP(hipGetLastError());
  return W4A8_OK;
}

}  // namespace w4a8
