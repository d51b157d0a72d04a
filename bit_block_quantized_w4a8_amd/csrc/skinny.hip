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
// all of K, with four groups of three waves; group q (waves q, 4 + q and
// 8 + q, which share SIMD q) owns a quarter of K, a range of consecutive
// blocks:
//   - the quantiser waves q and 4 + q load the group's activations first
//     (before any weight load enters the workgroup's memory pipeline), each
//     half of the tasks, and quantise them into the group's LDS region, four
//     blocks per step, each counting its finished steps in an LDS word;
//   - the MMA wave 8 + q streams the group's weights (8 bytes per lane, block
//     and tile) and weight scales, kSkAhead steps ahead of its MFMAs.  Per
//     block and tile it runs one MFMA with the activations as the A operand
//     (32 rows, those past M zero) and the weights as B (column = lane % 32,
//     the lane's 8 bytes giving 16 int4 values, times 16), accumulators
//     starting at the bits of 1.5 * 2^23 so the int32 result reads as a float;
//     then the GEMV's block step acc += RN(16 I sw) * (sx / 16) per row.
// A wave's loads are accepted in order and stall its instruction stream while
// the memory pipeline is full, so a wave that streams weights cannot also be
// the one that quantises: the split keeps the quantiser's arithmetic, the
// MFMAs and the block steps all under the weight stream.  The four MMA waves'
// partial sums are added through LDS in group order.  With the block-sum mode
// the int32 sums are exported instead.  K beyond 4 x kSkRound blocks runs in
// rounds separated by a workgroup barrier.
#include "kernels.hpp"

namespace w4a8 {
namespace {

constexpr int kSkThreads = 768;
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
constexpr int kSkPairs = 4;       // groups of (two quantiser waves, one MMA wave)
constexpr int kSkCols = 64;       // output columns per workgroup
constexpr int kSkStep = 4;        // K blocks per pipeline step
constexpr int kSkRound = 32;      // K blocks per pair and round
constexpr int kSkAhead = 2;       // steps of weights in flight ahead of the MFMAs
constexpr int kSkSpin = 1 << 22;  // bound of an MMA wave's wait for a step (never reached: the quantiser
                                  // wave of its pair is resident and waits for nothing)

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

// Memory step of pipeline step st: the ns steps of a round rotated by rot
// (steps past ns keep their place; they only reload the round's last block).
__device__ __forceinline__ int sk_step(int st, int rot, int ns) {
  if (st >= ns) return st;
  const int p = st + rot;
  return p < ns ? p : p - ns;
}

// MR: rows the kernel serves (8 or 16; M <= MR).
template <int MR, int MODE>
__global__ __launch_bounds__(kSkThreads) void skinny_kernel(SkinnyArgs a) {
  constexpr int RB = kSkRound;
  constexpr int S = RB / kSkStep;            // steps per round
  constexpr int XQ = RB * MR * 4 / 64;       // quantiser tasks of a group per lane and round: (row, block, quarter)
  constexpr int TPS = XQ / S;                // per step
  constexpr int XH = XQ / 2;                 // of one quantiser wave (tasks i with i % 2 == its half)
  constexpr int kRows = MR > 8 ? 8 : 4;      // accumulator entries per lane that can hold rows < MR
  __shared__ __align__(16) uint8_t codes[kSkPairs][RB][MR][32];
  __shared__ __align__(16) float sxl[kSkPairs][RB][MR];
  __shared__ __align__(16) uint16_t swl[kSkPairs][RB][kSkCols];
  // Steps finished by each quantiser wave (one word per wave: a count shared
  // by the two could reach a step's total while one of them still lags).
  __shared__ __align__(8) uint32_t ready[kSkPairs][2];
  static_assert(sizeof(codes) >= kSkPairs * 2 * kRows * 64 * sizeof(float), "reduction fits the codes");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = wave % kSkPairs;
  const bool mma = wave >= 2 * kSkPairs;      // wave-uniform role
  const int half = (wave / kSkPairs) & 1;     // a quantiser wave's tasks
  const int l32 = lane & 31, h = lane >> 5;
  const int M = a.M, K = a.K, N = a.N;
  const int nb = K / kBlock;
  const int bpp = nb / kSkPairs;              // blocks per pair (the host keeps nb % 8 == 0)
  const int n0 = blockIdx.x * kSkCols;
  // Workgroups on one XCD (blockIdx % 8 alike) share its L2 and all read the
  // same activations: each starts at its own quarter of K and its own step,
  // so that they do not meet on the same L2 lines at the same time.
  const int phase = blockIdx.x >> 3;
  const int pb0 = ((q + (phase >> 3)) % kSkPairs) * bpp;
  float* red = reinterpret_cast<float*>(&codes[0][0][0][0]);
  if (tid < 2 * kSkPairs) ready[tid / 2][tid % 2] = 0;

  float acc[2][kRows];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < kRows; ++r) acc[t][r] = 0.0f;

  // Each role runs its own loop over the rounds (one workgroup barrier per
  // round in both), so that neither role's registers are live in the other.
  if (!mma) {
    for (int j = 0, rb0 = 0; rb0 < bpp; ++j, rb0 += RB) {
      const int gn = min(RB, bpp - rb0);        // valid blocks of this round
      const int b0 = pb0 + rb0;                 // the round's first block
      const int ns = (gn + kSkStep - 1) / kSkStep, rot = phase % ns;
      // Task t = 64 i + lane is quarter t % 4 of block 2 p + (t / 4) % 2 of
      // row u % MR, u = t / 8, p = u / MR: one load instruction reads 128
      // consecutive bytes (two blocks) of each of 8 rows, and the tasks i of
      // step st cover blocks kSkStep st .. kSkStep st + kSkStep - 1 (in LDS;
      // in memory those of step sk_step(st, rot, ns)).
      uint4 xv[XH];
#pragma unroll
      for (int k = 0; k < XH; ++k) {
        const int t = 64 * (2 * k + half) + lane;
        const int u = t >> 3;
        const int st = k / (TPS / 2);
        const int bl = kSkStep * sk_step(st, rot, ns) + 2 * (u / MR) + ((t >> 2) & 1) - kSkStep * st;
        const int m = min(u % MR, M - 1);
        xv[k] = *reinterpret_cast<const uint4*>(a.x + static_cast<int64_t>(m) * K + (b0 + min(bl, gn - 1)) * kBlock +
                                                8 * (t & 3));
      }
      __syncthreads();  // (A) activations ahead of every weight load; the last round consumed
#pragma unroll
      for (int st = 0; st < S; ++st) {
        if (st < ns) {  // uniform
          // Codes: group g of a block's elements (8 g .. 8 g + 7) goes to
          // byte 8 * (0, 2, 1, 3)[g], so that lane half h of the MMA wave
          // reads element groups h and h + 2 as one 16-byte run.
#pragma unroll
          for (int k = TPS / 2 * st; k < TPS / 2 * (st + 1); ++k) {
            const int t = 64 * (2 * k + half) + lane;
            const int u = t >> 3, g = t & 3, bl = 2 * (u / MR) + ((t >> 2) & 1);
            float sx;
            bool near;
            uint2 qc = sk_quantize8(xv[k], u % MR < M, &sx, &near);
            if (near) qc = sk_quantize8_exact(xv[k], sx);
            const int slot = (g == 1) ? 2 : (g == 2) ? 1 : g;
            *reinterpret_cast<uint2*>(&codes[q][bl][u % MR][8 * slot]) = qc;
            if (g == 0) sxl[q][bl][u % MR] = sx * 0.0625f;
          }
          // The step's codes and scales are written (lgkmcnt(0)) before the
          // count rises.
          __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
          if (lane == 0)
            __hip_atomic_store(&ready[q][half], static_cast<uint32_t>(j * S + st + 1), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
    }
  } else {
    // The MMA wave issues before the quantiser waves of its SIMD: while it
    // waits for a turn, its next weight loads are not issued and the memory
    // pipeline runs dry.
    __builtin_amdgcn_s_setprio(3);
    for (int j = 0, rb0 = 0; rb0 < bpp; ++j, rb0 += RB) {
      const int gn = min(RB, bpp - rb0);
      const int b0 = pb0 + rb0;
      const int ns = (gn + kSkStep - 1) / kSkStep, rot = phase % ns;
      __syncthreads();  // (A)
      uint2 wv[RB][2];
      uint2 sv[S];
      auto issue = [&](int st) {
        // the step's weight scales (block kSkStep ps + lane / 16, columns
        // 4 (lane % 16) ..), then its weights
        const int pbl = kSkStep * sk_step(st, rot, ns);
        if (MODE == 0)
          sv[st] = *reinterpret_cast<const uint2*>(
              a.w_scales + static_cast<uint32_t>(b0 + min(pbl + lane / 16, gn - 1)) * N + n0 + 4 * (lane % 16));
#pragma unroll
        for (int r = kSkStep * st; r < kSkStep * (st + 1); ++r) {
          const int bl = b0 + min(pbl + r - kSkStep * st, gn - 1);
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const uint32_t off = static_cast<uint32_t>(bl * N + n0 + 32 * t + l32) * kPackedBytes + 8 * h;
            wv[r][t] = *reinterpret_cast<const uint2*>(a.packed_w + off);
          }
        }
      };
#pragma unroll
      for (int st = 0; st < kSkAhead; ++st) issue(st);
      v16i magic;
#pragma unroll
      for (int i = 0; i < 16; ++i) magic[i] = kMagicBits;
#pragma unroll
      for (int st = 0; st < S; ++st) {
        // Steps past the round's blocks load the last block again (clamped
        // indices) and skip their MFMAs: straight-line loads keep the
        // compiler's register assignment simple.
        if (st + kSkAhead < S) issue(st + kSkAhead);
        __builtin_amdgcn_sched_barrier(0);
        if (MODE == 0)
          *reinterpret_cast<uint2*>(&swl[q][kSkStep * st + lane / 16][4 * (lane % 16)]) = sv[st];
        if (st >= ns) continue;  // uniform: no blocks left (nothing published)
        const int pbl = kSkStep * sk_step(st, rot, ns) - kSkStep * st;  // memory block = LDS block + pbl
        const uint32_t want = static_cast<uint32_t>(j * S + st + 1);
        for (int spin = 0; spin < kSkSpin; ++spin) {
          const uint64_t both = __hip_atomic_load(reinterpret_cast<uint64_t*>(&ready[q][0]), __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_WORKGROUP);
          if (min(static_cast<uint32_t>(both), static_cast<uint32_t>(both >> 32)) >= want) break;
          __builtin_amdgcn_s_sleep(1);
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
        for (int r = kSkStep * st; r < kSkStep * (st + 1); ++r) {
          if (pbl + r < gn) {  // uniform
            v4i afrag = {0, 0, 0, 0};
            if (l32 < MR) afrag = *reinterpret_cast<const v4i*>(&codes[q][r][l32][16 * h]);
            // sx / 16 of accumulator rows 8 (j / 4) + 4 h + j % 4
            float sx16[kRows];
#pragma unroll
            for (int j4 = 0; j4 < kRows / 4; ++j4) {
              const float4 v = *reinterpret_cast<const float4*>(&sxl[q][r][8 * j4 + 4 * h]);
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
                for (int jj = 0; jj < kRows; ++jj) {
                  const int m = 8 * (jj / 4) + 4 * h + (jj % 4);
                  if (m < M) a.sums[(static_cast<int64_t>(m) * N + n) * nb + b0 + pbl + r] = (d[jj] - kMagicBits) >> 4;
                }
              } else {
                const float swf = half_bits_to_float(swl[q][r][32 * t + l32]);
                const float cst = swf * -kMagic;
#pragma unroll
                for (int jj = 0; jj < kRows; ++jj) {
                  const float tv = fmaf(__int_as_float(d[jj]), swf, cst);  // RN(16 I sw)
                  acc[t][jj] = fmaf(tv, sx16[jj], acc[t][jj]);
                }
              }
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if (MODE == 1) return;

  // Partial sums of the four MMA waves, added in pair order.
  __syncthreads();
  if (mma) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int jj = 0; jj < kRows; ++jj) red[((q * 2 + t) * kRows + jj) * 64 + lane] = acc[t][jj];
  }
  __syncthreads();
  for (int idx = tid; idx < 2 * kRows * 64; idx += kSkThreads) {
    const int ln = idx & 63, jj = (idx >> 6) % kRows, t = (idx >> 6) / kRows;
    const int m = 8 * (jj / 4) + 4 * (ln >> 5) + (jj % 4);
    if (m < M) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < kSkPairs; ++w) v += red[((w * 2 + t) * kRows + jj) * 64 + ln];
      a.out[static_cast<int64_t>(m) * N + n0 + 32 * t + (ln & 31)] = v;
    }
  }
}

template <int MR, int MODE>
int launch_mr(const SkinnyArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((skinny_kernel<MR, MODE>), dim3(a.N / kSkCols), dim3(kSkThreads), 0, stream, a);
  W4A8_HIP(hipGetLastError());
  return W4A8_OK;
}

}  // namespace

bool skinny_supported(int M, int K, int N) {
  return M >= 1 && M <= 16 && K % (kBlock * 8) == 0 && N % kSkCols == 0;
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
