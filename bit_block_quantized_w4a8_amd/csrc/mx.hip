// MX variant of the block-32 linear: MXFP4 weights x MXFP8 activations on
// gfx950's block-scaled matrix instruction (v_mfma_scale_f32_32x32x64_f8f6f4).
//
// The pages fix 4-bit weights in blocks of 32 (ML Drift explainer on
// tech.dede.sh, section "Stage-aware optimization for large language
// models").  This variant keeps both and takes its number formats from the
// OCP Microscaling (MX) v1.0 specification: a block of 32 values shares an
// E8M0 scale 2^(c - 127) with c = floor(log2(max |v|)) - emax + 127 (emax = 8
// for FP8 E4M3 elements, 2 for FP4 E2M1), and each value / scale is rounded to
// the element format, nearest with ties to even, saturating at the largest
// normal (448, 6).  The matrix instruction applies both block scales itself,
// so the prefill product needs no per-block fp32 epilogue.
//
// Operand layout of v_mfma_scale_f32_32x32x64_f8f6f4 with A = E4M3 (rows m)
// and B = E2M1 (columns n), K = 64 (two scale blocks) per instruction, as
// measured on gfx950 with one-hot and random operands:
//   A: lane l, byte p holds row l % 32, k = 32 (p / 16) + 16 (l / 32) + p % 16;
//   B: lane l, nibble q (low nibble first) holds column l % 32, k = 32 (l / 32) + q;
//   scales: lane l's A (B) scale byte covers row (column) l % 32, k block l / 32;
//   D: lane l, register r holds row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
//
// Layouts in memory (all K-block-major so that a lane's bytes are contiguous):
//   weights  packed [K/32][N][16]: byte j of (block b, column n) holds
//            element 32b + 2j in its low nibble and 32b + 2j + 1 in its high;
//            scales [K/32][N] E8M0 bytes;
//   activations (library staging) codes [K/32][M_pad][32] E4M3 bytes,
//            scales [K/32][M_pad] E8M0 bytes (rows M .. M_pad-1 zero).
// A K step (two blocks) of a 128 x 128 tile is then eight contiguous runs:
// codes and weights of each block, and the scales of each block.
#include "kernels.hpp"
#include "lds_dma.hpp"

namespace w4a8 {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kE4M3 = 0;   // matrix-instruction format code of FP8 E4M3
constexpr int kE2M1 = 4;   // matrix-instruction format code of FP4 E2M1

// floor(log2 a) of a positive finite fp32 value, from its exponent field.
__device__ __forceinline__ int floor_log2(float a) {
  const uint32_t bits = __float_as_uint(a);
  const int e = static_cast<int>((bits >> 23) & 0xFF);
  if (e != 0) return e - 127;
  return -126 - (__builtin_clz(bits & 0x7FFFFF) - 9);  // subnormal fp32 (not reached from fp16)
}

// Magnitude code of a >= 0 (already clamped to the largest normal) in a
// sign-magnitude minifloat with MB mantissa bits and exponent bias BIAS:
// nearest, ties to even.  Below 2^(1 - BIAS) the step is 2^(1 - BIAS - MB).
template <int MB, int BIAS>
__device__ __forceinline__ uint32_t minifloat_code(float a) {
  constexpr int kMinExp = 1 - BIAS;
  if (a < __builtin_ldexpf(1.0f, kMinExp)) {
    // integer multiple of the subnormal step (2^MB is the smallest normal code)
    return static_cast<uint32_t>(__builtin_rintf(__builtin_ldexpf(a, MB - kMinExp)));
  }
  const int e = floor_log2(a);
  const float frac = __builtin_ldexpf(a, -e) - 1.0f;            // exact, in [0, 1)
  uint32_t mq = static_cast<uint32_t>(__builtin_rintf(__builtin_ldexpf(frac, MB)));
  int ee = e;
  if (mq == (1u << MB)) {
    mq = 0;
    ++ee;
  }
  return (static_cast<uint32_t>(ee + BIAS) << MB) | mq;
}

__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const float a = fminf(fabsf(v), 448.0f);
  const uint32_t mag = minifloat_code<3, 7>(a);
  return (v < 0.0f && mag != 0 ? 0x80u : 0u) | (mag < 0x7Eu ? mag : 0x7Eu);
}

__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fminf(fabsf(v), 6.0f);
  const uint32_t mag = minifloat_code<1, 1>(a);
  return (v < 0.0f && mag != 0 ? 0x8u : 0u) | (mag < 0x7u ? mag : 0x7u);
}

// Max of |v| over an aligned quad of lanes (DPP quad permutes).
__device__ __forceinline__ float quad_amax(float a) {
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0xB1, 0xF, 0xF, true)));
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0x4E, 0xF, 0xF, true)));
  return a;
}

// E8M0 scale code of a block from its max magnitude (0 for an all-zero block)
// and the power of two 2^-shared that maps the block onto the element grid.
template <int EMAX>
__device__ __forceinline__ uint32_t block_scale(float amax, float* inv_scale) {
  if (!(amax > 0.0f)) {
    *inv_scale = 0.0f;
    return 0u;
  }
  const int shared = floor_log2(amax) - EMAX;
  *inv_scale = __builtin_ldexpf(1.0f, -shared);
  return static_cast<uint32_t>(shared + 127);
}

// One aligned quad of lanes per (row, block): lane g of the quad converts
// elements 8g .. 8g+7.  MXFP8 activations into staging (see the file comment).
__global__ __launch_bounds__(256) void mx_quantize_act_kernel(const uint16_t* __restrict__ x, int M, int M_pad,
                                                              int K, uint8_t* __restrict__ codes,
                                                              uint8_t* __restrict__ scales) {
  // x of the grid: rows (four lanes each); y: blocks (no runtime division).
  const int tx = blockIdx.x * blockDim.x + threadIdx.x;
  if (tx >= 4 * M_pad) return;  // whole quads in or out (4 | 256)
  const int nb = K / kBlock;
  const int g = tx & 3;
  const int64_t m = tx >> 2;
  for (int64_t b = blockIdx.y; b < nb; b += gridDim.y) {
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (m < M) unpack_half8(*reinterpret_cast<const uint4*>(x + m * K + b * kBlock + 8 * g), v);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = quad_amax(amax);
    float inv;
    const uint32_t sc = block_scale<8>(amax, &inv);
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i >> 2] |= e4m3_code(v[i] * inv) << (8 * (i & 3));  // v * 2^-shared is exact
    *reinterpret_cast<uint2*>(codes + (b * M_pad + m) * kBlock + 8 * g) = make_uint2(w[0], w[1]);
    if (g == 0) scales[b * M_pad + m] = static_cast<uint8_t>(sc);
  }
}

// MXFP4 weights: one aligned quad per (column n, block b) of w [N][K].
__global__ __launch_bounds__(256) void mx_pack_kernel(const uint16_t* __restrict__ w, int K, int N,
                                                      uint8_t* __restrict__ packed, uint8_t* __restrict__ scales) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int nb = K / kBlock;
  if (t >= static_cast<int64_t>(N) * nb * 4) return;
  const int g = static_cast<int>(t & 3);
  const int64_t q = t >> 2;
  const int64_t n = q % N;
  const int64_t b = q / N;
  float v[8];
  unpack_half8(*reinterpret_cast<const uint4*>(w + n * K + b * kBlock + 8 * g), v);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = quad_amax(amax);
  float inv;
  const uint32_t sc = block_scale<2>(amax, &inv);
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) word |= e2m1_code(v[i] * inv) << (4 * i);
  *reinterpret_cast<uint32_t*>(packed + (b * N + n) * 16 + 4 * g) = word;
  if (g == 0) scales[b * N + n] = static_cast<uint8_t>(sc);
}

// GEMM: four waves per workgroup, each wave a 64 x 64 output tile (2 x 2
// instruction tiles).  WK = 1: the waves form 2 x 2 over a 128 x 128 tile.
// WK = 4 (shapes whose 128 x 128 tiles would leave CUs idle): the four waves
// share one 64 x 64 tile and take interleaved K steps, and their accumulators
// are added through LDS in wave order.  Operands stream from global memory
// (L2) straight into registers, kPre K steps ahead; each K step of 64 is one
// block-scaled instruction per 32 x 32 tile.  Rows and columns beyond M and N
// are clamped on load and skipped on store.
constexpr int kMxThreads = 256;
constexpr int kMxRowPad = 128;   // staging rows are padded to this multiple

struct MxFrag {
  v8i a[2];      // A rows of the wave's two m tiles: 32 E4M3 bytes each
  int b[2][4];   // B columns of its two n tiles: 32 E2M1 nibbles each
  uint32_t sa[2], sb[2];
};

template <int WK>
__global__ __launch_bounds__(kMxThreads) void mx_gemm_kernel(const uint8_t* __restrict__ codes,
                                                             const uint8_t* __restrict__ ascale,
                                                             const uint8_t* __restrict__ packed,
                                                             const uint8_t* __restrict__ wscale, int M, int M_pad,
                                                             int K, int N, int tiles_m, float* __restrict__ out) {
  constexpr int kTileM = WK == 1 ? 128 : 64;
  constexpr int kTileN = WK == 1 ? 128 : 64;
  __shared__ float red[WK > 1 ? (WK - 1) * 4 * 16 * 64 : 1];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  // Consecutive workgroups share a weight tile (all m tiles of one n tile)
  // and are dealt round-robin over the 8 XCDs: map them to one XCD.
  const int tiles = gridDim.x;
  const int id = (tiles & 7) == 0 ? (blockIdx.x & 7) * (tiles >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  const int tn = id / tiles_m;
  const int tm = id % tiles_m;
  const int m_base = tm * kTileM + (WK == 1 ? (wave & 1) * 64 : 0);
  const int n_base = tn * kTileN + (WK == 1 ? (wave >> 1) * 64 : 0);
  const int wk = WK == 1 ? 0 : wave;
  const int steps = K / 64;

  int rows[2], cols[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    rows[i] = min(m_base + 32 * i + l32, M_pad - 1);
    cols[i] = min(n_base + 32 * i + l32, N - 1);
  }
  auto load = [&](int s, MxFrag& f) __attribute__((always_inline)) {
    const int b0 = 2 * s;  // blocks b0 (bytes 0..15) and b0 + 1 (bytes 16..31), half h of each
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint8_t* r0 = codes + (static_cast<int64_t>(b0) * M_pad + rows[i]) * kBlock + 16 * h;
      const uint4 lo = *reinterpret_cast<const uint4*>(r0);
      const uint4 hi = *reinterpret_cast<const uint4*>(r0 + static_cast<int64_t>(M_pad) * kBlock);
      f.a[i][0] = lo.x; f.a[i][1] = lo.y; f.a[i][2] = lo.z; f.a[i][3] = lo.w;
      f.a[i][4] = hi.x; f.a[i][5] = hi.y; f.a[i][6] = hi.z; f.a[i][7] = hi.w;
      f.sa[i] = ascale[static_cast<int64_t>(b0 + h) * M_pad + rows[i]];
      const uint4 wv = *reinterpret_cast<const uint4*>(packed + (static_cast<int64_t>(b0 + h) * N + cols[i]) * 16);
      f.b[i][0] = wv.x; f.b[i][1] = wv.y; f.b[i][2] = wv.z; f.b[i][3] = wv.w;
      f.sb[i] = wscale[static_cast<int64_t>(b0 + h) * N + cols[i]];
    }
  };

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // This wave's K steps: wk, wk + WK, ...; the loads run kPre of them ahead
  // (clamped to the wave's last step, so every wave issues the same loads).
  const int my_steps = steps > wk ? (steps - wk + WK - 1) / WK : 0;
  auto step_of = [&](int i) { return wk + WK * min(i, my_steps - 1); };
  constexpr int kPre = 3;
  MxFrag fr[kPre + 1];
  if (my_steps > 0) {  // uniform
#pragma unroll
    for (int p = 0; p < kPre; ++p) load(step_of(p), fr[p]);
    for (int i0 = 0; i0 < my_steps; i0 += kPre + 1) {
#pragma unroll
      for (int u = 0; u <= kPre; ++u) {
        const int i = i0 + u;
        if (i < my_steps) {  // uniform
          load(step_of(i + kPre), fr[(u + kPre) % (kPre + 1)]);
          const MxFrag& f = fr[u];
#pragma unroll
          for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
              const v8i bv = {f.b[b][0], f.b[b][1], f.b[b][2], f.b[b][3], 0, 0, 0, 0};
              acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[a], bv, acc[a][b], kE4M3, kE2M1, 0,
                                                                          f.sa[a], 0, f.sb[b]);
            }
        }
      }
    }
  }

  if constexpr (WK > 1) {
    // Waves 1 .. WK-1 hand their tiles to wave 0, which adds them in wave order.
    if (wave > 0) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) red[(((wave - 1) * 4 + a * 2 + b) * 16 + r) * 64 + lane] = acc[a][b][r];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 1; w < WK; ++w)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[a][b][r] += red[(((w - 1) * 4 + a * 2 + b) * 16 + r) * 64 + lane];
  }

  // D: lane l, register r -> row 8 (r / 4) + 4 h + r % 4 of the tile, column l % 32.
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int n = n_base + 32 * b + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m_base + 32 * a + 8 * (r / 4) + 4 * h + r % 4;
        if (m < M && n < N) out[static_cast<int64_t>(m) * N + n] = acc[a][b][r];
      }
    }
}

// GEMM with LDS staging: four waves (2 x 2, each 64 x 64) on a 128 x 128 tile.
// A K step's operands (eight runs, 12800 bytes) are copied straight into LDS
// with global_load_lds_dwordx4, 64 chunks of 16 bytes per instruction, into a
// ring of three stages filled two steps ahead; each wave waits on its own
// copies and one barrier per step publishes a stage, so every operand byte
// crosses from L2 once per workgroup instead of once per wave.
struct MxStage {
  static constexpr int kA0 = 0;        // codes of block 2s, rows 0..127 (32 B each)
  static constexpr int kA1 = 4096;     // codes of block 2s+1
  static constexpr int kB0 = 8192;     // weights of block 2s, columns 0..127 (16 B each)
  static constexpr int kB1 = 10240;    // weights of block 2s+1
  static constexpr int kSA = 12288;    // activation scales, blocks 2s and 2s+1 (128 B each)
  static constexpr int kSB = 12544;    // weight scales, blocks 2s and 2s+1
  static constexpr int kChunks = 800;  // 12800 bytes
  static constexpr int kGroups = 13;   // DMA instructions per stage (the last one half padding)
  static constexpr int kBytes = kGroups * 1024;
};

__global__ __launch_bounds__(kMxThreads) void mx_gemm_lds_kernel(const uint8_t* __restrict__ codes,
                                                                 const uint8_t* __restrict__ ascale,
                                                                 const uint8_t* __restrict__ packed,
                                                                 const uint8_t* __restrict__ wscale, int M,
                                                                 int M_pad, int K, int N, int tiles_m,
                                                                 float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t st0[MxStage::kBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st1[MxStage::kBytes];
  __shared__ __attribute__((aligned(16))) uint8_t st2[MxStage::kBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int tiles = gridDim.x;
  const int id = (tiles & 7) == 0 ? (blockIdx.x & 7) * (tiles >> 3) + (blockIdx.x >> 3) : blockIdx.x;
  const int tn = id / tiles_m;
  const int tm = id % tiles_m;
  const int m0 = tm * 128;
  const int n0 = tn * 128;
  const int steps = K / 64;
  const int last = steps - 1;

  // This lane's chunk of each of the wave's DMA instructions (groups wave,
  // wave + 4, ...): source of step 0 and the source's advance per step.
  constexpr int kL = (MxStage::kGroups + 3) / 4;  // 4 for wave 0, 3 for the others
  const int my_loads = (MxStage::kGroups - wave + 3) / 4;
  const uint8_t* src[kL];
  uint32_t adv[kL];
#pragma unroll
  for (int i = 0; i < kL; ++i) {
    const int c = min((wave + 4 * i) * 64 + lane, MxStage::kChunks - 1);  // padding lanes repeat chunk 799
    if (c < 256) {
      src[i] = codes + (static_cast<int64_t>(m0) * kBlock) + 16 * c;
      adv[i] = 2u * static_cast<uint32_t>(M_pad) * kBlock;
    } else if (c < 512) {
      src[i] = codes + (static_cast<int64_t>(M_pad) + m0) * kBlock + 16 * (c - 256);
      adv[i] = 2u * static_cast<uint32_t>(M_pad) * kBlock;
    } else if (c < 768) {
      const int blk = (c - 512) / 128;
      const int col = min(n0 + (c - 512) % 128, N - 1);
      src[i] = packed + (static_cast<int64_t>(blk) * N + col) * 16;
      adv[i] = 2u * static_cast<uint32_t>(N) * 16;
    } else if (c < 784) {
      const int blk = (c - 768) / 8;
      src[i] = ascale + static_cast<int64_t>(blk) * M_pad + m0 + 16 * ((c - 768) % 8);
      adv[i] = 2u * static_cast<uint32_t>(M_pad);
    } else {
      const int blk = (c - 784) / 8;
      src[i] = wscale + static_cast<int64_t>(blk) * N + min(n0 + 16 * ((c - 784) % 8), N - 16);
      adv[i] = 2u * static_cast<uint32_t>(N);
    }
  }
  auto dma = [&](uint8_t* st, int s) __attribute__((always_inline)) {
    const uint32_t ss = static_cast<uint32_t>(min(s, last));
#pragma unroll
    for (int i = 0; i < kL; ++i)
      if (i < my_loads) lds::dma16(src[i] + static_cast<uint64_t>(ss) * adv[i], st + (wave + 4 * i) * 1024);
  };

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int wm = wave & 1, wn = wave >> 1;
  auto compute = [&](const uint8_t* st) __attribute__((always_inline)) {
    v8i a[2];
    uint32_t sa[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = wm * 64 + 32 * i + l32;
      const uint4 lo = *reinterpret_cast<const uint4*>(st + MxStage::kA0 + r * 32 + 16 * h);
      const uint4 hi = *reinterpret_cast<const uint4*>(st + MxStage::kA1 + r * 32 + 16 * h);
      a[i][0] = lo.x; a[i][1] = lo.y; a[i][2] = lo.z; a[i][3] = lo.w;
      a[i][4] = hi.x; a[i][5] = hi.y; a[i][6] = hi.z; a[i][7] = hi.w;
      sa[i] = st[MxStage::kSA + 128 * h + r];
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = wn * 64 + 32 * j + l32;
      const uint4 wv = *reinterpret_cast<const uint4*>(st + MxStage::kB0 + h * 2048 + c * 16);
      const v8i bv = {static_cast<int>(wv.x), static_cast<int>(wv.y), static_cast<int>(wv.z), static_cast<int>(wv.w),
                      0, 0, 0, 0};
      const uint32_t sb = st[MxStage::kSB + 128 * h + c];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], bv, acc[i][j], kE4M3, kE2M1, 0, sa[i], 0,
                                                                    sb);
    }
  };

  // Step s: wait for this wave's copies of step s, publish the stage, refill
  // the stage read last step with step s + 2, multiply step s.  At most two
  // steps' copies are in flight, so vmcnt(my_loads) leaves exactly step s + 1's.
#define W4A8_MX_STEP(CUR, REFILL, S)                                 \
  do {                                                               \
    if (my_loads == kL) lds::wait_vmcnt<kL>();                       \
    else lds::wait_vmcnt<kL - 1>();                                  \
    lds::stage_barrier();                                            \
    dma((REFILL), (S) + 2);                                          \
    if ((S) < steps) compute(CUR);                                   \
  } while (0)
  dma(st0, 0);
  dma(st1, 1);
  for (int s = 0; s < steps; s += 3) {
    W4A8_MX_STEP(st0, st2, s + 0);
    W4A8_MX_STEP(st1, st0, s + 1);
    W4A8_MX_STEP(st2, st1, s + 2);
  }
#undef W4A8_MX_STEP
  lds::wait_vmcnt<0>();  // copies past the end are still in flight

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + 32 * j + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + 32 * i + 8 * (r / 4) + 4 * h + r % 4;
        if (m < M && n < N) out[static_cast<int64_t>(m) * N + n] = acc[i][j][r];
      }
    }
}

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

}  // namespace

int mx_m_pad(int M) { return (M + kMxRowPad - 1) / kMxRowPad * kMxRowPad; }

size_t mx_scratch_bytes(int M, int K) {
  const size_t m_pad = mx_m_pad(M);
  return align256(m_pad * K) + align256(m_pad * (K / kBlock));  // codes, then scales [K/32][M_pad]
}

int launch_mx_quantize_act(const uint16_t* x, int M, int M_pad, int K, uint8_t* codes, uint8_t* scales,
                           hipStream_t stream) {
  const int nb = K / kBlock;
  const dim3 grid((4 * M_pad + 255) / 256, nb < 65535 ? nb : 65535);
  hipLaunchKernelGGL(mx_quantize_act_kernel, grid, dim3(256), 0, stream, x, M, M_pad, K, codes, scales);
  W4A8_HIP(hipGetLastError());
  return W4A8_OK;
}

int launch_mx_pack(const uint16_t* w, int K, int N, uint8_t* packed, uint8_t* scales, hipStream_t stream) {
  const int64_t threads = static_cast<int64_t>(N) * (K / kBlock) * 4;
  hipLaunchKernelGGL(mx_pack_kernel, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, stream, w,
                     K, N, packed, scales);
  W4A8_HIP(hipGetLastError());
  return W4A8_OK;
}

int launch_mx_linear(const uint16_t* x, const uint8_t* packed, const uint8_t* wscales, int M, int K, int N,
                     float* out, Scratch* sc, hipStream_t stream) {
  const int m_pad = mx_m_pad(M);
  int rc = require_scratch(sc, mx_scratch_bytes(M, K));
  if (rc != W4A8_OK) return rc;
  uint8_t* codes = static_cast<uint8_t*>(sc->work);
  uint8_t* ascale = codes + align256(static_cast<size_t>(m_pad) * K);
  rc = launch_mx_quantize_act(x, M, m_pad, K, codes, ascale, stream);
  if (rc != W4A8_OK) return rc;
  // 128 x 128 tiles when they give two workgroups per CU, else K split over
  // the four waves of each 64 x 64 tile.
  constexpr int kCUs = 256;
  const int big = (m_pad / 128) * ((N + 127) / 128);
  if (big >= 2 * kCUs) {
    hipLaunchKernelGGL(mx_gemm_lds_kernel, dim3(big), dim3(kMxThreads), 0, stream, codes, ascale, packed, wscales, M,
                       m_pad, K, N, m_pad / 128, out);
  } else {
    const int tiles_m = m_pad / 64;
    hipLaunchKernelGGL(mx_gemm_kernel<4>, dim3(tiles_m * ((N + 63) / 64)), dim3(kMxThreads), 0, stream, codes, ascale,
                       packed, wscales, M, m_pad, K, N, tiles_m, out);
  }
  W4A8_HIP(hipGetLastError());
  return W4A8_OK;
}

}  // namespace w4a8
