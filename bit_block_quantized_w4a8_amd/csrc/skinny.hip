// Small-batch decode kernel: a few token rows (M = 3 .. 16) on the int8 matrix
// instruction, with the decode GEMV's memory pattern.
//
// The decode GEMV forms one int8 dot product per row and weight block, so its
// arithmetic grows with M; the prefill GEMM stages pre-quantised activations
// and reads each weight tile for 32 or more rows.  Between them (the pages'
// stage split: ML Drift explainer on tech.dede.sh, section "Stage-aware
// optimization for large language models"), this kernel streams every weight
// once, as the GEMV does, and forms the block sums of all rows at once on
// v_mfma_i32_32x32x32_i8, as the GEMM does.
//
// Work split: a workgroup owns 64 output columns (two 32-column tiles) over
// all of K; its 8 waves split K into eight ranges of consecutive blocks.  Each
// wave
//   1. loads its rows' activations for its K range (first, so that waiting
//      for them never waits for weights: a wave's loads retire in order), then
//      its weights (8 bytes per lane, block and tile) and weight scales;
//   2. quantises its activations into its own LDS region, per 32-element block
//      (method below), eight blocks at a time;
//   3. per block and tile: one MFMA with the activations as the A operand (32
//      rows, those past M zero) and the weights as B (column = lane % 32, the
//      lane's 8 bytes giving 16 int4 values, times 16), accumulators starting
//      at the bits of 1.5 * 2^23 so the int32 result reads as a float; then
//      the GEMV's block step acc += RN(16 I sw) * (sx / 16) per row.
// The eight waves' partial sums are added through LDS in wave order.  With
// the block-sum mode the int32 sums are exported instead.
#include "kernels.hpp"

namespace w4a8 {
namespace {

constexpr int kSkThreads = 512;
// Every workgroup quantises all M x K activations (the weights of its columns
// need all of them), so the quantiser is written for few instructions:
//
//   amax   the max of the fp16 magnitudes as 16-bit integers (for finite
//          values the bit patterns with the sign cleared order as the
//          magnitudes do), over the lane's 8 values with packed 16-bit maxima
//          and over the quad with two DPP steps, then widened to fp32;
//   sx     fp32(amax / 127) from q0 = amax * c, e = fma(-q0, 127, amax),
//          sx = fma(e, c, q0) with c = fp32(1/127): equal to the IEEE
//          quotient for every positive fp16 amax (checked over all 31743);
//   code   t = fma(x, r, 1.5 * 2^23) with r = rcp(sx) rounds the exact product
//          x * r to the nearest integer, ties to even, and the low byte of t's
//          bits is that integer as an int8 code.  v_rcp_f32 is within 1 ulp,
//          so x * r is within |x / sx| * 2^-23 <= 1.52e-5 of x / sx, and the
//          IEEE quotient fp32(x / sx) within 7.6e-6; where x * r lies further
//          than kSkTieWindow = 2^-14 from the nearest k + 1/2 (measured by
//          d = fma(x, r, -k), exact to 2^-25), both round to the same integer.
//          Lanes with an element inside the window recompute their codes from
//          the IEEE quotient (about one task in twenty has one).
// |x / sx| <= 127.00003, so no code needs clamping; amax = 0 gives sx = 0 and
// r = 0, hence zero codes.
constexpr float kSkTieWindow = 1.0f / 16384.0f;
constexpr int kSkWaves = 8;
constexpr int kSkCols = 64;       // output columns per workgroup
constexpr int kSkGroup = 4;       // K blocks per pipeline step of a wave

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

struct SkinnyArgs {
  const uint16_t* x;       // fp16 [M][K]
  const uint8_t* packed_w;
  const uint16_t* w_scales;
  int M, K, N;
  float* out;              // MODE 0: fp32 [M][N]
  int32_t* sums;           // MODE 1: int32 [M][N][K/32]
};

__device__ __forceinline__ float sk_half(uint32_t w, int hi) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(hi ? w >> 16 : w)));
}

// Codes of the lane's 8 elements (a quarter of a block held by an aligned quad
// of lanes) and the block scale; *near is set where a code must be recomputed.
// `real` is false for rows past M (uniform over the quad): zero codes, sx = 0.
__device__ __forceinline__ uint2 sk_quantize8(uint4 xv, bool real, float* sx_out, bool* near) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  const uint32_t w[4] = {xv.x, xv.y, xv.z, xv.w};
  u16x2 m = __builtin_bit_cast(u16x2, w[0] & 0x7FFF7FFFu);
#pragma unroll
  for (int i = 1; i < 4; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
  uint32_t mb = m.x > m.y ? m.x : m.y;
  mb = max(mb, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(mb), 0xB1, 0xF, 0xF, true)));
  mb = max(mb, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(mb), 0x4E, 0xF, 0xF, true)));
  const float a = real ? sk_half(mb, 0) : 0.0f;
  const float c = 1.0f / 127.0f;
  const float q0 = a * c;
  const float sx = fmaf(fmaf(-q0, 127.0f, a), c, q0);
  const float r = a > 0.0f ? __builtin_amdgcn_rcpf(sx) : 0.0f;
  uint32_t t[8];
  float dm = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float x = sk_half(w[i / 2], i & 1);
    const float ti = fmaf(x, r, kMagic);
    dm = fmaxf(dm, fabsf(fmaf(x, r, kMagic - ti)));
    t[i] = __float_as_uint(ti);
  }
  *near = dm >= 0.5f - kSkTieWindow;
  *sx_out = sx;
  return make_uint2(__builtin_amdgcn_perm(t[1], t[0], 0x0C0C0400u) | __builtin_amdgcn_perm(t[3], t[2], 0x04000C0Cu),
                    __builtin_amdgcn_perm(t[5], t[4], 0x0C0C0400u) | __builtin_amdgcn_perm(t[7], t[6], 0x04000C0Cu));
}

// The same codes from the IEEE quotient, round half to even.
__device__ __forceinline__ uint2 sk_quantize8_exact(uint4 xv, float sx) {
  const uint32_t w[4] = {xv.x, xv.y, xv.z, xv.w};
  uint32_t packed[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = static_cast<int>(__builtin_rintf(sk_half(w[i / 2], i & 1) / sx));
    packed[i / 4] |= (static_cast<uint32_t>(q) & 0xFFu) << (8 * (i % 4));
  }
  return make_uint2(packed[0], packed[1]);
}

// MR: rows the kernel serves (8 or 16; M <= MR).  R: K blocks per wave per
// round of weight loads (8 or 16).
template <int MR, int R, int MODE>
__global__ __launch_bounds__(kSkThreads) void skinny_kernel(SkinnyArgs a) {
  static_assert(R % kSkGroup == 0, "pipeline steps");
  constexpr int kTasks = MR * R * 4;        // quantisation tasks of a wave's round: (row, block, quarter)
  constexpr int XQ = kTasks / 64;           // per lane
  constexpr int TPG = XQ / (R / kSkGroup);  // per lane and pipeline step
  constexpr int kRows = MR > 8 ? 8 : 4;     // accumulator entries per lane that can hold rows < MR
  // LDS: a wave's codes of R blocks x MR rows (32 bytes each), its sx / 16
  // per (block, row) and its weight scales per (block, column); the
  // cross-wave reduction reuses the codes.
  __shared__ __align__(16) uint8_t codes[kSkWaves][R][MR][32];
  __shared__ __align__(16) float sxl[kSkWaves][R][MR];
  __shared__ __align__(16) uint16_t swl[kSkWaves][R][kSkCols];
  static_assert(sizeof(codes) >= kSkWaves * 2 * kRows * 64 * sizeof(float), "reduction fits the codes");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int M = a.M, K = a.K, N = a.N;
  const int nb = K / kBlock;
  const int bpw = nb / kSkWaves;            // blocks per wave (the host keeps nb % 8 == 0)
  const int n0 = blockIdx.x * kSkCols;
  const int wb0 = wave * bpw;
  float* red = reinterpret_cast<float*>(&codes[0][0][0][0]);

  float acc[2][kRows];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < kRows; ++r) acc[t][r] = 0.0f;
  v16i magic;
#pragma unroll
  for (int i = 0; i < 16; ++i) magic[i] = kMagicBits;

  for (int g0 = 0; g0 < bpw; g0 += R) {
    const int gn = min(R, bpw - g0);        // valid blocks of this round
    // 1. Activations and weight scales of the round.  Task t = 64 i + lane is
    //    quarter t % 4 of block 2 p + (t / 4) % 2 of row u % MR, u = t / 8,
    //    p = u / MR: one load instruction reads 128 consecutive bytes (two
    //    blocks) of each of 8 rows, and tasks i of step s cover blocks
    //    kSkGroup s .. kSkGroup s + kSkGroup - 1.
    uint4 xv[XQ];
#pragma unroll
    for (int i = 0; i < XQ; ++i) {
      const int t = 64 * i + lane;
      const int u = t >> 3;
      const int m = min(u % MR, M - 1), bl = min(2 * (u / MR) + ((t >> 2) & 1), gn - 1);
      xv[i] = *reinterpret_cast<const uint4*>(a.x + static_cast<int64_t>(m) * K + (wb0 + g0 + bl) * kBlock + 8 * (t & 3));
    }
    // R blocks x 64 columns of fp16 scales, 16-byte piece e = lane + 64 i
    // holding block e / 8, columns 8 (e % 8) .. 8 (e % 8) + 7 (two named
    // registers rather than an array, which the compiler left in memory).
    uint4 sv0 = {}, sv1 = {};
    if (MODE == 0) {
      const uint32_t col = static_cast<uint32_t>(n0 + 8 * (lane % 8));
      sv0 = *reinterpret_cast<const uint4*>(a.w_scales + static_cast<uint32_t>(wb0 + g0 + min(lane / 8, gn - 1)) * N + col);
      if (R == 16)
        sv1 = *reinterpret_cast<const uint4*>(a.w_scales + static_cast<uint32_t>(wb0 + g0 + min(8 + lane / 8, gn - 1)) * N + col);
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2. Pipeline over steps of kSkGroup blocks: issue step s's weights,
    //    quantise step s's activations into LDS, then run step s - 1's MFMAs.
    //    A wave's loads are accepted in order and stall its instruction stream
    //    while the memory pipeline is full, so work placed after all of the
    //    round's loads would wait for nearly all of them; interleaved, the
    //    quantiser and the MFMAs run while later weights are in flight.
    uint2 wv[R][2];
#pragma unroll
    for (int st = 0; st <= R / kSkGroup; ++st) {
      if (st < R / kSkGroup) {
#pragma unroll
        for (int r = kSkGroup * st; r < kSkGroup * (st + 1); ++r) {
          const int bl = wb0 + g0 + min(r, gn - 1);
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const uint32_t off = static_cast<uint32_t>(bl * N + n0 + 32 * t + l32) * kPackedBytes + 8 * h;
            wv[r][t] = *reinterpret_cast<const uint2*>(a.packed_w + off);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (st == 0 && MODE == 0) {
          *reinterpret_cast<uint4*>(&swl[wave][lane / 8][8 * (lane % 8)]) = sv0;
          if (R == 16) *reinterpret_cast<uint4*>(&swl[wave][8 + lane / 8][8 * (lane % 8)]) = sv1;
        }
        // Codes: group q of a block's elements (8 q .. 8 q + 7) goes to byte
        // 8 * (0, 2, 1, 3)[q], so that lane half h reads element groups h and
        // h + 2 as one 16-byte run.
#pragma unroll
        for (int i = TPG * st; i < TPG * (st + 1); ++i) {
          const int t = 64 * i + lane;
          const int u = t >> 3, q = t & 3, bl = 2 * (u / MR) + ((t >> 2) & 1);
          float sx;
          bool near;
          uint2 qc = sk_quantize8(xv[i], u % MR < M, &sx, &near);
          if (near) qc = sk_quantize8_exact(xv[i], sx);
          const int slot = (q == 1) ? 2 : (q == 2) ? 1 : q;
          *reinterpret_cast<uint2*>(&codes[wave][bl][u % MR][8 * slot]) = qc;
          if (q == 0) sxl[wave][bl][u % MR] = sx * 0.0625f;
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_sched_barrier(0);
      }
      if (st == 0) continue;

      // 3. MFMA per block and tile of step st - 1, then the block step.
#pragma unroll
      for (int r = kSkGroup * (st - 1); r < kSkGroup * st; ++r) {
        if (r < gn) {  // uniform
          v4i afrag = {0, 0, 0, 0};
          if (l32 < MR) afrag = *reinterpret_cast<const v4i*>(&codes[wave][r][l32][16 * h]);
          // sx / 16 of accumulator rows 8 (j / 4) + 4 h + j % 4
          float sx16[kRows];
#pragma unroll
          for (int j4 = 0; j4 < kRows / 4; ++j4) {
            const float4 v = *reinterpret_cast<const float4*>(&sxl[wave][r][8 * j4 + 4 * h]);
            sx16[4 * j4] = v.x;
            sx16[4 * j4 + 1] = v.y;
            sx16[4 * j4 + 2] = v.z;
            sx16[4 * j4 + 3] = v.w;
          }
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            v4i bfrag;
            bfrag[0] = static_cast<int>(low_nibbles_x16(wv[r][t].x));
            bfrag[1] = static_cast<int>(low_nibbles_x16(wv[r][t].y));
            bfrag[2] = static_cast<int>(high_nibbles_x16(wv[r][t].x));
            bfrag[3] = static_cast<int>(high_nibbles_x16(wv[r][t].y));
            const v16i d = __builtin_amdgcn_mfma_i32_32x32x32_i8(afrag, bfrag, magic, 0, 0, 0);
            const int n = n0 + 32 * t + l32;
            if (MODE == 1) {
#pragma unroll
              for (int j = 0; j < kRows; ++j) {
                const int m = 8 * (j / 4) + 4 * h + (j % 4);
                if (m < M) a.sums[(static_cast<int64_t>(m) * N + n) * nb + wb0 + g0 + r] = (d[j] - kMagicBits) >> 4;
              }
            } else {
              const float swf = half_bits_to_float(swl[wave][r][32 * t + l32]);
              const float cst = swf * -kMagic;
#pragma unroll
              for (int j = 0; j < kRows; ++j) {
                const float tv = fmaf(__int_as_float(d[j]), swf, cst);  // RN(16 I sw)
                acc[t][j] = fmaf(tv, sx16[j], acc[t][j]);
              }
            }
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_wave_barrier();  // the next round rewrites this wave's LDS
  }
  if (MODE == 1) return;

  // Partial sums of the eight waves, added in wave order.
  __syncthreads();
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int j = 0; j < kRows; ++j) red[((wave * 2 + t) * kRows + j) * 64 + lane] = acc[t][j];
  __syncthreads();
  for (int idx = tid; idx < 2 * kRows * 64; idx += kSkThreads) {
    const int ln = idx & 63, j = (idx >> 6) % kRows, t = (idx >> 6) / kRows;
    const int m = 8 * (j / 4) + 4 * (ln >> 5) + (j % 4);
    if (m < M) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < kSkWaves; ++w) v += red[((w * 2 + t) * kRows + j) * 64 + ln];
      a.out[static_cast<int64_t>(m) * N + n0 + 32 * t + (ln & 31)] = v;
    }
  }
}

template <int MR, int MODE>
int launch_mr(const SkinnyArgs& a, hipStream_t stream) {
  const int bpw = a.K / kBlock / kSkWaves;
  const dim3 grid(a.N / kSkCols);
  if (bpw <= 8) hipLaunchKernelGGL((skinny_kernel<MR, 8, MODE>), grid, dim3(kSkThreads), 0, stream, a);
  else hipLaunchKernelGGL((skinny_kernel<MR, 16, MODE>), grid, dim3(kSkThreads), 0, stream, a);
  W4A8_HIP(hipGetLastError());
  return W4A8_OK;
}

}  // namespace

bool skinny_supported(int M, int K, int N) {
  return M >= 1 && M <= 16 && K % (kBlock * kSkWaves) == 0 && N % kSkCols == 0;
}

int launch_skinny(const uint16_t* x, const uint8_t* packed_w, const uint16_t* w_scales, int M, int K, int N,
                  float* out, int32_t* sums, hipStream_t stream) {
  if (!skinny_supported(M, K, N)) return hip_fail(hipErrorInvalidValue, "small-batch kernel: shape outside its limits");
  if (static_cast<int64_t>(K / kBlock) * N * kPackedBytes >= (int64_t{1} << 32))
    return hip_fail(hipErrorInvalidValue, "small-batch kernel: weights beyond 4 GiB");
  const SkinnyArgs a{x, packed_w, w_scales, M, K, N, out, sums};
  if (sums) return M <= 8 ? launch_mr<8, 1>(a, stream) : launch_mr<16, 1>(a, stream);
  return M <= 8 ? launch_mr<8, 0>(a, stream) : launch_mr<16, 0>(a, stream);
}

}  // namespace w4a8
