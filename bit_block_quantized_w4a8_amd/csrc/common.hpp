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

// Scratch memory of the kernels: the library's own per-device buffers
// (w4a8_init, w4a8_reserve_scratch) or a view over another region of device
// memory.  No launcher allocates: each checks that `work` is large enough.
struct Scratch {
  void* base = nullptr;
  size_t bytes = 0;
  uint32_t* tickets = nullptr;       // split-K / attention completion counters, self-resetting
  int n_tickets = 0;
  unsigned long long* slots = nullptr;  // argmax keys [kMaxArgmaxRows][kArgmaxSpread], reset by the finaliser
  void* work = nullptr;              // staging: quantised activations, split-K partials
  size_t work_bytes = 0;
};
constexpr int kMaxTickets = 1 << 16;
constexpr int kMaxArgmaxRows = 64;
// Argmax keys of one row are spread over this many slots (tile % spread), so
// the per-workgroup atomic maxima of a launch do not all meet on one address.
constexpr int kArgmaxSpread = 64;
// The library scratch of the current device (W4A8_ENOINIT before w4a8_init).
int library_scratch(Scratch** out);
// W4A8_EINVAL, with a message naming the bytes needed, if sc's work area is
// smaller than work_bytes.
int require_scratch(const Scratch* sc, size_t work_bytes);

// ------------------------------------------------------------- device side
__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<unsigned short>(h)));
}
// fp32 -> fp16 bits, round to nearest even.
__device__ __forceinline__ uint16_t float_to_half_bits(float v) {
  return __builtin_bit_cast(unsigned short, static_cast<_Float16>(v));
}

// Quantise one 32-element activation block held by an aligned quad of lanes,
// eight consecutive elements per lane (lane % 4 = g holds elements 8g .. 8g+7).
// Returns the eight int8 codes packed little-endian into two dwords and writes
// the block scale sx = fp32(amax / 127) to *sx_out (0 for an all-zero block).
//
// The codes equal round_half_even(fp32(x / sx)) exactly.  amax is exact (a max
// of exact fp16 -> fp32 widenings, in any order) and sx is the IEEE division.
// Each code is first estimated as y = x * rcp(sx): v_rcp_f32 is accurate to
// 1 ulp, so |y - x/sx| <= |x/sx| * (2^-23 + 2^-24) < 2.5e-5 and the IEEE
// quotient is within 7.6e-6 of x/sx, since |x/sx| <= 127.5.  Where y is further
// than kTieWindow = 2^-12 from the nearest k + 1/2, both round to the same
// integer; otherwise the code is recomputed from the IEEE division.  The
// recomputation is rare (about 2 * 2^-12 of random inputs), so most elements
// cost a multiply, a rounding and a compare instead of a division.
constexpr float kTieWindow = 1.0f / 4096.0f;

// Max over the 4 lanes of an aligned quad (DPP quad permutes, no LDS traffic).
__device__ __forceinline__ float quad_max(float a) {
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0xB1, 0xF, 0xF, true)));  // lane ^ 1
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0x4E, 0xF, 0xF, true)));  // lane ^ 2
  return a;
}

// The codes of eight elements of a block whose max-abs is `a` and whose scale
// is sx = fp32(a / 127), by the method above.
__device__ __forceinline__ uint2 quantize8_codes(const float* x, float a, float sx) {
  if (!(a > 0.0f)) return make_uint2(0u, 0u);
  const float r = __builtin_amdgcn_rcpf(sx);
  float q[8];
  bool near_tie = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float y = x[i] * r;
    q[i] = __builtin_rintf(y);
    near_tie |= fabsf(y - q[i]) >= 0.5f - kTieWindow;
  }
  if (near_tie) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float y = x[i] * r;
      if (fabsf(y - q[i]) >= 0.5f - kTieWindow) q[i] = __builtin_rintf(x[i] / sx);
    }
  }
  uint32_t packed[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float c = fminf(fmaxf(q[i], -127.0f), 127.0f);
    packed[i >> 2] |= (static_cast<uint32_t>(static_cast<int>(c)) & 0xFFu) << (8 * (i & 3));
  }
  return make_uint2(packed[0], packed[1]);
}

__device__ __forceinline__ uint2 quantize8_group4(const float* x, float* sx_out) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(x[i]));
  a = quad_max(a);
  const float sx = a / 127.0f;
  *sx_out = sx;
  return quantize8_codes(x, a, sx);
}

// Quantises group e (elements 8e .. 8e+7, held in v) of row m into the GEMM
// staging layout (gemm.hip): codes at qxs + b * m_pad * 32, 16-byte slot
// ((m / 32) * 2 + h) * 32 + m % 32 with h = g % 2, byte offset 8 * (g / 2), for
// block b = e / 4 and group g = e % 4 (elements 8g .. 8g+7 of the block belong
// at byte 8 * (0, 2, 1, 3)[g] of the row's 32 codes); the block scale goes to
// sxs[b * m_pad + m].  Called by an aligned quad of lanes per block.
__device__ __forceinline__ void quantize_to_staging(const float* v, int64_t m, int64_t e, int64_t m_pad,
                                                    uint8_t* __restrict__ qxs, float* __restrict__ sxs) {
  float scale;
  const uint2 codes = quantize8_group4(v, &scale);
  const int g = static_cast<int>(e & 3);
  const int64_t b = e >> 2;
  const int64_t row_slot = ((m >> 5) * 2 + (g & 1)) * 32 + (m & 31);
  *reinterpret_cast<uint2*>(qxs + b * m_pad * kBlock + row_slot * 16 + 8 * (g >> 1)) = codes;
  if (g == 0) sxs[b * m_pad + m] = scale;
}

// fp16 bits of fp16(fp32(a * b)): the product is rounded to fp32 first, then
// to fp16.  The product is made opaque to the optimiser because the backend
// otherwise folds the multiply and the conversion into one mixed-precision
// instruction (v_fma_mixlo_f16) that rounds the exact product to fp16 once;
// near an fp16 rounding midpoint the two differ by one fp16 unit.
__device__ __forceinline__ uint16_t half_of_product(float a, float b) {
  float p = a * b;
  asm("" : "+v"(p));
  return float_to_half_bits(p);
}

// 1 / sqrt(mean(x^2) + eps) of a row of H fp32 values, from the row's sum of
// squares ss formed in fp64.  Each square of an fp32 value is exact in fp64
// and a sum of H of them, in any order, is within H * 2^-53 of the exact sum
// (relative; 2^-42 for H = 2048).  Kernels that add the squares in different
// orders (the normalising GEMV prologue, the glue kernels) therefore get the
// same fp32 result unless the exact value lies that close to an fp32
// rounding boundary (2^-23 apart), and the fp16 inputs they hand to a linear
// agree bit for bit.
__device__ __forceinline__ float rms_inverse(double ss, int H, float eps) {
  return static_cast<float>(1.0 / sqrt(ss / static_cast<double>(H) + static_cast<double>(eps)));
}
// Square of an fp32 value added to an fp64 sum (the square is exact).
__device__ __forceinline__ double add_square(double acc, float v) {
  const double d = static_cast<double>(v);
  return fma(d, d, acc);
}

// The eight fp16 values of a 16-byte load, widened to fp32 (exact).
__device__ __forceinline__ void unpack_half8(uint4 v, float* x) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = half_bits_to_float(w[i] & 0xFFFFu);
    x[2 * i + 1] = half_bits_to_float(w[i] >> 16);
  }
}

// int4 nibbles -> int8 bytes holding 16 * value (two's complement nibble moved
// to the top of each byte): low nibbles of a packed dword, and high nibbles.
__device__ __forceinline__ uint32_t low_nibbles_x16(uint32_t w) { return (w << 4) & kNibbleMask; }
__device__ __forceinline__ uint32_t high_nibbles_x16(uint32_t w) { return w & kNibbleMask; }

// Partial results handed between workgroups of one launch: agent-scope
// accesses go to the device-coherent level, past the issuing CU's L1.
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<uint32_t*>(const_cast<float*>(p)),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

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
