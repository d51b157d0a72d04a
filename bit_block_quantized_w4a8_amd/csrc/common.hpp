// Shared host and device helpers of the W4A8 block-32 library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/w4a8.h"

namespace w4a8 {

constexpr int kBlock = 32;             // inputs per quantisation block
constexpr int kPackedBytes = 16;       // bytes of one (block, column) weight group
constexpr uint32_t kNibbleMask = 0xF0F0F0F0u;

// 1.5 * 2^23 as fp32 bits.  Adding a signed integer |v| < 2^22 to these bits
// gives the fp32 number 1.5 * 2^23 + v exactly; the int8 dot products start
// their integer accumulators here so the sum can be read back as a float
// without a conversion instruction.
constexpr int32_t kMagicBits = 0x4B400000;
constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23

// ---------------------------------------------------------------- host side
void set_error(const char* fmt, ...);
int hip_fail(hipError_t e, const char* what);

#define W4A8_HIP(call)                                   \
  do {                                                   \
    hipError_t e_ = (call);                              \
    if (e_ != hipSuccess) return ::w4a8::hip_fail(e_, #call); \
  } while (0)

// Library scratch of the current device.
struct Scratch {
  void* base = nullptr;
  size_t bytes = 0;
  uint32_t* tickets = nullptr;       // split-K / argmax completion counters, self-resetting
  unsigned long long* slots = nullptr;  // argmax keys, self-resetting
  void* work = nullptr;              // staging: quantised activations, split-K partials
  size_t work_bytes = 0;
};
constexpr int kMaxTickets = 1 << 16;
constexpr int kMaxArgmaxRows = 64;
int scratch_for(size_t work_bytes, Scratch** out);  // grows `work` if needed

// ------------------------------------------------------------- device side
__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<unsigned short>(h)));
}

// Quantise one 32-element activation block held by 8 consecutive lanes, four
// consecutive elements per lane (lane % 8 = g holds elements 4g .. 4g+3).
// Returns the four int8 codes packed little-endian into one dword and writes
// the block scale sx = fp32(amax / 127) to *sx_out (0 for an all-zero block).
// amax is exact (max of exact fp16 -> fp32 widenings, in any order); x / sx is
// the IEEE division and rintf rounds half to even, so the codes do not depend
// on the lane or reduction order.
__device__ __forceinline__ uint32_t quantize4_group8(float x0, float x1, float x2, float x3,
                                                     float* sx_out) {
  float a = fmaxf(fmaxf(fabsf(x0), fabsf(x1)), fmaxf(fabsf(x2), fabsf(x3)));
  a = fmaxf(a, __shfl_xor(a, 1));
  a = fmaxf(a, __shfl_xor(a, 2));
  a = fmaxf(a, __shfl_xor(a, 4));
  const float sx = a / 127.0f;
  *sx_out = sx;
  if (!(a > 0.0f)) return 0u;
  const float lo = -127.0f, hi = 127.0f;
  const int q0 = static_cast<int>(fminf(fmaxf(__builtin_rintf(x0 / sx), lo), hi));
  const int q1 = static_cast<int>(fminf(fmaxf(__builtin_rintf(x1 / sx), lo), hi));
  const int q2 = static_cast<int>(fminf(fmaxf(__builtin_rintf(x2 / sx), lo), hi));
  const int q3 = static_cast<int>(fminf(fmaxf(__builtin_rintf(x3 / sx), lo), hi));
  return (static_cast<uint32_t>(q0) & 0xFFu) | ((static_cast<uint32_t>(q1) & 0xFFu) << 8) |
         ((static_cast<uint32_t>(q2) & 0xFFu) << 16) | (static_cast<uint32_t>(q3) << 24);
}

// The four fp16 values of an 8-byte load, widened to fp32 (exact).
__device__ __forceinline__ void unpack_half4(uint2 v, float* x) {
  x[0] = half_bits_to_float(v.x & 0xFFFFu);
  x[1] = half_bits_to_float(v.x >> 16);
  x[2] = half_bits_to_float(v.y & 0xFFFFu);
  x[3] = half_bits_to_float(v.y >> 16);
}

// int4 nibbles -> int8 bytes holding 16 * value (two's complement nibble moved
// to the top of each byte): low nibbles of a packed dword, and high nibbles.
__device__ __forceinline__ uint32_t low_nibbles_x16(uint32_t w) { return (w << 4) & kNibbleMask; }
__device__ __forceinline__ uint32_t high_nibbles_x16(uint32_t w) { return w & kNibbleMask; }

// Total order on finite floats as unsigned keys, -0.0 mapped to +0.0.
__device__ __forceinline__ uint32_t orderable_key(float v) {
  uint32_t b = __float_as_uint(v);
  if ((b & 0x7FFFFFFFu) == 0) b = 0;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
// argmax key: larger value wins, then lower column index.
__device__ __forceinline__ unsigned long long argmax_key(float v, uint32_t col) {
  return (static_cast<unsigned long long>(orderable_key(v)) << 32) |
         static_cast<unsigned long long>(0xFFFFFFFFu - col);
}

}  // namespace w4a8
